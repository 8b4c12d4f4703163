"""Shared pieces of the GPU parity tests: seeded inputs, the oracle side, the HIP side and the
comparison at the tolerance the target sets (max |err| <= 2e-2 * max |ref| and cosine >= 0.9999,
per tensor and per ragged segment)."""

import numpy as np

from attention_backward_fmha_amd import inputs as I

TOL_MAX = 2e-2
TOL_COS = 0.9999


def seq_offsets(lengths):
    return I.seqstart(lengths)


def make_inputs(seed, *, B=None, Sq=None, Sk=None, lens_q=None, lens_k=None, Hq, Hkv, d_qk, d_v,
                sigmas=(1, 1, 1, 1)):
    """Batch mode when lens_q is None.  Returns dict of float32 bf16-representable arrays."""
    if lens_q is None:
        shapes = [(B, Sq, Hq, d_qk), (B, Sk, Hkv, d_qk), (B, Sk, Hkv, d_v), (B, Sq, Hq, d_v)]
    else:
        tq, tk = int(sum(lens_q)), int(sum(lens_k))
        shapes = [(tq, Hq, d_qk), (tk, Hkv, d_qk), (tk, Hkv, d_v), (tq, Hq, d_v)]
    return I.draw(seed, shapes, sigmas)


def oracle_forward(x, *, scale, mask, window=(-1, -1), sq=None, sk=None):
    import oracle
    o, lse = oracle.forward(x["q"], x["k"], x["v"], scale=scale, mask_type=mask,
                            window_left=window[0], window_right=window[1], seqstart_q=sq,
                            seqstart_k=sk)
    return o, lse


def oracle_backward(x, *, scale, mask, window=(-1, -1), sq=None, sk=None):
    import oracle
    return oracle.backward(x["q"], x["k"], x["v"], x["do"], scale=scale, mask_type=mask,
                           window_left=window[0], window_right=window[1], seqstart_q=sq,
                           seqstart_k=sk)


def to_dev_bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()


def to_dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def run_gpu(x, o, lse, *, scale, mask, window=(-1, -1), sq=None, sk=None, deterministic=True,
            dq_acc_dtype="fp32", tune=None):
    """Round O to bf16 and LSE to fp32 as the forward would store them, run the library."""
    import torch
    import attention_backward_fmha_amd as F
    q, k, v, do = (to_dev_bf16(x[n]) for n in ("q", "k", "v", "do"))
    od = to_dev_bf16(I.round_bf16(o.astype(np.float32)))
    ld = to_dev_f32(lse.astype(np.float32))
    kw = {}
    if sq is not None:
        kw = dict(cu_seqlens_q=torch.from_numpy(np.asarray(sq, np.int32)).cuda(),
                  cu_seqlens_k=torch.from_numpy(np.asarray(sk, np.int32)).cuda(),
                  cu_seqlens_q_host=np.asarray(sq, np.int32),
                  cu_seqlens_k_host=np.asarray(sk, np.int32))
    dq, dk, dv = F.bwd(q, k, v, od, ld, do, scale=scale, mask_type=mask, window=window,
                       deterministic=deterministic, dq_acc_dtype=dq_acc_dtype, tune=tune, **kw)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))


def metrics(got, ref):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    mref = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    ng, nr = np.linalg.norm(got), np.linalg.norm(ref)
    if nr == 0.0 and ng == 0.0:
        cos = 1.0
    elif nr == 0.0 or ng == 0.0:
        cos = 0.0
    else:
        cos = float(got @ ref / (ng * nr))
    return err, mref, cos


def assert_close(name, got, ref):
    assert np.all(np.isfinite(got)), "%s has non-finite values" % name
    err, mref, cos = metrics(got, ref)
    if mref == 0.0:
        assert err == 0.0, "%s: reference is zero but max|got| = %g" % (name, err)
        return
    assert err <= TOL_MAX * mref, "%s: max|err| %.3g > %.3g * max|ref| (%.3g)" % (name, err, TOL_MAX, mref)
    assert cos >= TOL_COS, "%s: cosine %.6f < %.4f" % (name, cos, TOL_COS)


def assert_grads_close(got, ref, sq=None, sk=None, label=""):
    names = ("dq", "dk", "dv")
    for n, g, r in zip(names, got, ref):
        assert_close(label + n, g, r)
    if sq is not None:
        for b in range(len(sq) - 1):
            for n, g, r, s in zip(names, got, ref, (sq, sk, sk)):
                a0, a1 = int(s[b]), int(s[b + 1])
                if a1 > a0:
                    assert_close("%s%s[segment %d]" % (label, n, b), g[a0:a1], r[a0:a1])



def single_key_floors(x, o, scale, allowed, group):
    """Error floors of dQ and dK where every query row has at most one allowed key.

    There dS = P (dP - D) vanishes exactly, so the exact dQ and dK are 0.  But the backward
    gets O rounded to bf16 and computes D_i = dO_i . O~_i, so each such row leaves
    delta_i = |dO_i . (O_i - O~_i)| in dS.  This gives |dQ_i| <= scale * delta_i * max|K| and
    |dK_j| <= scale * (sum over the rows i that attend j and the query heads of j's group of
    delta_i) * max|Q|.  x, o: one segment, arrays [rows, H, d]; allowed: [Lq, Lk] bool.
    Returns the floors, twice the bound plus fp32 noise."""
    ot = I.round_bf16(np.asarray(o, np.float32)).astype(np.float64)
    delta = np.abs((np.asarray(x["do"], np.float64) * (np.asarray(o, np.float64) - ot)).sum(-1))  # [Lq, Hq]
    kmax = float(np.abs(x["k"]).max()) if np.size(x["k"]) else 0.0
    qmax = float(np.abs(x["q"]).max()) if np.size(x["q"]) else 0.0
    fq = 2 * scale * (float(delta.max()) if delta.size else 0.0) * kmax + 1e-5
    hq = delta.shape[1] if delta.ndim == 2 else 1
    per_key = np.zeros(allowed.shape[1])
    for h in range(hq):
        per_key += allowed.T.astype(np.float64) @ delta[:, h]  # summed over the group's heads too
    fk = 2 * scale * (float(per_key.max()) if per_key.size else 0.0) * qmax + 1e-5
    return fq, fk


def assert_vanishing(name, got, floor):
    assert np.all(np.isfinite(got)), name
    m = float(np.abs(got).max()) if np.size(got) else 0.0
    assert m <= floor, "%s: exact value 0 (one key per row), max|got| = %.3g > floor %.3g" % (name, m, floor)
