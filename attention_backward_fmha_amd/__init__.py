"""MI355X (gfx950) fused multi-head attention backward.

Thin Python surface over the C ABI of ``include/fmha_bwd.h``: every step of the computation
runs in the library's HIP kernels; torch tensors only carry device memory and the stream.

    dq, dk, dv = attention_backward_fmha_amd.bwd(q, k, v, o, lse, do, mask_type=1)

Batch (BSHD) tensors are [B, S, H, d] with LSE [B, Hq, Sq]; group (THD, ragged) tensors are
[T, H, d] with LSE [Hq, T] and ``cu_seqlens_q``/``cu_seqlens_k`` offsets (B+1 int32).  Padded
THD adds ``cu_seqlens_q_padded``/``cu_seqlens_k_padded``: segment b's rows start at physical
row padded[b] and the rest of its slot (up to padded[b+1]) is padding, left untouched.
``dq_acc_dtype="bf16"`` (with ``deterministic=False``) accumulates dQ with packed bf16 atomic
adds instead of fp32 ones: about half the atomic traffic, less accurate dQ.
``bias`` (batch mode): a bf16 [1|B, 1|Hq, Sq, Sk] tensor added to the scaled logits;
``bwd(..., bias=bias, bias_grad=True)`` also returns dbias, shaped like the bias.
``dropout_p``, ``philox_seed``, ``philox_offset``: dropout on the probabilities of O = P V
(forward) and in dV, dP (backward), with the Philox keep mask of ``include/fmha_bwd.h``; the
backward must get the forward's values.
``tune`` (tests and tuning): a dict of layout overrides ``kernel`` (KERNEL_FOUR_WAVE or
KERNEL_WIDE), ``tile_m``, ``tiles_per_item``, ``kv_parts``; absent keys leave the plan's choice.
"""

import numpy as np

from . import _lib
from ._lib import (  # noqa: F401
    MASK_NONE, MASK_CAUSAL_TOP_LEFT, MASK_CAUSAL_BOTTOM_RIGHT, MASK_WINDOW, DQ_ACC_FP32, DQ_ACC_BF16,
    KERNEL_AUTO, KERNEL_FOUR_WAVE, KERNEL_WIDE,
    STAGE_DOT, STAGE_MAIN, STAGE_REDUCE, STAGE_ALL,
    Args, PlanInfo, FmhaError, status_string, workspace_size, plan_query,
)


class BwdCall:
    """An argument struct plus the Python objects whose memory it points at."""

    def __init__(self, args, keep):
        self.args = args
        self.keep = keep

    def workspace_size(self):
        return _lib.workspace_size(self.args)

    def plan(self):
        return _lib.plan_query(self.args)

    def prepare(self, ws, stream):
        _lib.prepare_workspace(self.args, ws.data_ptr(), ws.numel() * ws.element_size(), stream)

    def run(self, ws, stream, stages=STAGE_ALL):
        _lib.run(self.args, ws.data_ptr(), ws.numel() * ws.element_size(), stream, stages)

    def run_noalloc(self, stream):
        """prepare + run in the library's static scratch (fmha_bwd_run_noalloc): no workspace
        argument and no device allocation."""
        _lib.run_noalloc(self.args, stream)


def _strides(t, group):
    if t is None:
        return (0, 0, 0)
    if t.numel() == 0:  # nothing is addressed; report dense strides
        st = [1] * t.dim()
        for i in range(t.dim() - 2, -1, -1):
            st[i] = st[i + 1] * max(1, t.shape[i + 1])
    else:
        st = t.stride()
    if st[-1] != 1:
        raise ValueError("the head dimension must be contiguous")
    if group:
        return (0, st[0], st[1])
    return (st[0], st[1], st[2])


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _check_lse(lse, shape):
    """The ABI reads LSE with a unit sequence stride from device memory."""
    if tuple(lse.shape) != tuple(shape):
        raise ValueError("lse must have shape %s, got %s" % (tuple(shape), tuple(lse.shape)))
    if not lse.is_cuda:
        raise ValueError("lse must be a device tensor")
    if lse.numel() > 0 and lse.shape[-1] > 1 and lse.stride(-1) != 1:
        raise ValueError("lse must have a unit stride along the sequence")


def make_call(q, k, v, o, lse, do, dq, dk, dv, *, scale=None, mask_type=MASK_NONE,
              window=(-1, -1), deterministic=True, cu_seqlens_q=None, cu_seqlens_k=None,
              cu_seqlens_q_host=None, cu_seqlens_k_host=None, max_seqlen_q=None,
              max_seqlen_k=None, cu_seqlens_q_padded=None, cu_seqlens_k_padded=None,
              cu_seqlens_q_padded_host=None, cu_seqlens_k_padded_host=None, dq_acc_dtype="fp32",
              bias=None, dbias=None, dropout_p=0.0, philox_seed=0, philox_offset=0, tune=None):
    """Fill the C argument struct from tensors (no device work)."""
    group = cu_seqlens_q is not None
    d_qk = q.shape[-1]
    d_v = v.shape[-1]
    keep = [q, k, v, o, lse, do, dq, dk, dv]
    a = Args()
    if group:
        if cu_seqlens_q_host is None:
            cu_seqlens_q_host = cu_seqlens_q.cpu().numpy()
        if cu_seqlens_k_host is None:
            cu_seqlens_k_host = cu_seqlens_k.cpu().numpy()
        hq_ = np.ascontiguousarray(cu_seqlens_q_host, dtype=np.int32)
        hk_ = np.ascontiguousarray(cu_seqlens_k_host, dtype=np.int32)
        keep += [hq_, hk_, cu_seqlens_q, cu_seqlens_k]
        B = len(hq_) - 1
        lq = np.diff(hq_)
        lk = np.diff(hk_)
        a.B = B
        a.Sq = int(max_seqlen_q if max_seqlen_q is not None else (lq.max() if B else 0))
        a.Sk = int(max_seqlen_k if max_seqlen_k is not None else (lk.max() if B else 0))
        a.seqstart_q_host = hq_.ctypes.data
        a.seqstart_k_host = hk_.ctypes.data
        a.seqstart_q_dev = cu_seqlens_q.data_ptr()
        a.seqstart_k_dev = cu_seqlens_k.data_ptr()
        a.Hq, a.Hkv = q.shape[1], k.shape[1]
        _check_lse(lse, (a.Hq, q.shape[0]))
        a.lse_stride[0] = 0
        a.lse_stride[1] = lse.stride(0)
        for side, dev_t, host in (("q", cu_seqlens_q_padded, cu_seqlens_q_padded_host),
                                  ("k", cu_seqlens_k_padded, cu_seqlens_k_padded_host)):
            if dev_t is None:
                continue
            if host is None:
                host = dev_t.cpu().numpy()
            h_ = np.ascontiguousarray(host, dtype=np.int32)
            keep += [h_, dev_t]
            setattr(a, "seqstart_%s_padded_host" % side, h_.ctypes.data)
            setattr(a, "seqstart_%s_padded_dev" % side, dev_t.data_ptr())
    else:
        a.B, a.Sq, a.Hq = q.shape[0], q.shape[1], q.shape[2]
        a.Sk, a.Hkv = k.shape[1], k.shape[2]
        _check_lse(lse, (a.B, a.Hq, a.Sq))
        a.lse_stride[0] = lse.stride(0)
        a.lse_stride[1] = lse.stride(1)
    a.d_qk, a.d_v = d_qk, d_v
    a.scale = float(scale if scale is not None else 1.0 / np.sqrt(d_qk))
    a.mask_type = int(mask_type)
    a.window_left, a.window_right = (int(window[0]), int(window[1]))
    a.deterministic = 1 if deterministic else 0
    if dq_acc_dtype not in ("fp32", "bf16"):
        raise ValueError("dq_acc_dtype must be 'fp32' or 'bf16'")
    a.dq_acc_dtype = DQ_ACC_BF16 if dq_acc_dtype == "bf16" else DQ_ACC_FP32
    for key, val in (tune or {}).items():
        if key not in ("kernel", "tile_m", "tiles_per_item", "kv_parts"):
            raise ValueError("unknown tune key %r" % key)
        setattr(a, "tune_" + key, int(val))
    a.p_drop = float(dropout_p)
    a.philox_seed = int(philox_seed) & (2**64 - 1)
    a.philox_offset = int(philox_offset) & (2**64 - 1)
    if bias is not None:
        if bias.dim() != 4 or bias.stride(-1) != 1:
            raise ValueError("bias must be [1|B, 1|Hq, Sq, Sk] with contiguous columns")
        keep.append(bias)
        a.bias = bias.data_ptr()
        a.bias_b, a.bias_h = bias.shape[0], bias.shape[1]
        for i in range(3):
            a.bias_stride[i] = bias.stride(i)
    if dbias is not None:
        if bias is None or dbias.shape != bias.shape or dbias.stride(-1) != 1:
            raise ValueError("dbias must have the bias's shape, with contiguous columns")
        keep.append(dbias)
        a.dbias = dbias.data_ptr()
        for i in range(3):
            a.dbias_stride[i] = dbias.stride(i)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", do), ("lse", lse),
                    ("dq", dq), ("dk", dk), ("dv", dv)):
        setattr(a, name, _ptr(t))
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o),
                    ("do_stride", do), ("dq_stride", dq), ("dk_stride", dk), ("dv_stride", dv)):
        s = _strides(t, group)
        arr = getattr(a, name)
        arr[0], arr[1], arr[2] = s
    return BwdCall(a, keep)


def bwd(q, k, v, o, lse, do, *, scale=None, mask_type=MASK_NONE, window=(-1, -1),
        deterministic=True, cu_seqlens_q=None, cu_seqlens_k=None, cu_seqlens_q_host=None,
        cu_seqlens_k_host=None, max_seqlen_q=None, max_seqlen_k=None, cu_seqlens_q_padded=None,
        cu_seqlens_k_padded=None, cu_seqlens_q_padded_host=None, cu_seqlens_k_padded_host=None,
        workspace=None, out=None, dq_acc_dtype="fp32", bias=None, bias_grad=False, dropout_p=0.0,
        philox_seed=0, philox_offset=0, tune=None):
    """Gradients (dq, dk, dv) of softmax attention, and dbias when ``bias_grad``; see the
    module docstring for layouts."""
    import torch

    for t in (q, k, v, o, do):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q, k, v, o and do must be bfloat16 CUDA tensors")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    if out is not None:  # caller-provided (dq, dk, dv), e.g. to keep padding rows
        dq, dk, dv = out
    else:
        dq = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        dk = torch.empty(k.shape, dtype=torch.bfloat16, device=k.device)
        dv = torch.empty(v.shape, dtype=torch.bfloat16, device=v.device)
    dbias = None
    if bias_grad:
        if bias is None:
            raise ValueError("bias_grad needs a bias")
        dbias = torch.empty(bias.shape, dtype=torch.bfloat16, device=bias.device)
    call = make_call(q, k, v, o, lse, do, dq, dk, dv, scale=scale, mask_type=mask_type,
                     window=window, deterministic=deterministic, cu_seqlens_q=cu_seqlens_q,
                     cu_seqlens_k=cu_seqlens_k, cu_seqlens_q_host=cu_seqlens_q_host,
                     cu_seqlens_k_host=cu_seqlens_k_host, max_seqlen_q=max_seqlen_q,
                     max_seqlen_k=max_seqlen_k, cu_seqlens_q_padded=cu_seqlens_q_padded,
                     cu_seqlens_k_padded=cu_seqlens_k_padded,
                     cu_seqlens_q_padded_host=cu_seqlens_q_padded_host,
                     cu_seqlens_k_padded_host=cu_seqlens_k_padded_host, dq_acc_dtype=dq_acc_dtype,
                     bias=bias, dbias=dbias, dropout_p=dropout_p, philox_seed=philox_seed,
                     philox_offset=philox_offset, tune=tune)
    nbytes = call.workspace_size()
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    call.prepare(workspace, stream)
    call.run(workspace, stream)
    if bias_grad:
        return dq, dk, dv, dbias
    return dq, dk, dv


def fwd(q, k, v, *, scale=None, mask_type=MASK_NONE, window=(-1, -1), cu_seqlens_q=None,
        cu_seqlens_k=None, cu_seqlens_q_host=None, cu_seqlens_k_host=None, max_seqlen_q=None,
        max_seqlen_k=None, cu_seqlens_q_padded=None, cu_seqlens_k_padded=None,
        cu_seqlens_q_padded_host=None, cu_seqlens_k_padded_host=None, bias=None, dropout_p=0.0,
        philox_seed=0, philox_offset=0):
    """Forward (o, lse) on the device, in the layouts ``bwd`` takes: o like q with d_v columns,
    lse [B, Hq, Sq] (batch) or [Hq, T] (group)."""
    import torch

    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q, k and v must be bfloat16 CUDA tensors")
    o = torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=torch.bfloat16, device=q.device)
    if cu_seqlens_q is not None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    else:
        lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
    call = make_call(q, k, v, o, lse, None, None, None, None, scale=scale, mask_type=mask_type,
                     window=window, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
                     cu_seqlens_q_host=cu_seqlens_q_host, cu_seqlens_k_host=cu_seqlens_k_host,
                     max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
                     cu_seqlens_q_padded=cu_seqlens_q_padded, cu_seqlens_k_padded=cu_seqlens_k_padded,
                     cu_seqlens_q_padded_host=cu_seqlens_q_padded_host,
                     cu_seqlens_k_padded_host=cu_seqlens_k_padded_host, bias=bias,
                     dropout_p=dropout_p, philox_seed=philox_seed, philox_offset=philox_offset)
    _lib.fwd_run(call.args, torch.cuda.current_stream(q.device).cuda_stream)
    return o, lse
