"""fp64 CPU oracle of softmax attention: forward (O, LSE) and exact backward (dQ, dK, dV).

Test infrastructure only (see the package docstring): the product library never imports it.

What is computed, and which passage each piece follows
------------------------------------------------------
The pages (three pull-request pages about AMD's FMHA backward) treat the backward as a black
box; the arithmetic below is the textbook definition of scaled-dot-product softmax
attention and of its gradient, which is what a fused attention backward reaches exactly (up
to rounding order).

* Mask encoding -- "Update AITER subcommit and refactor internal AITER/CK FA API usage"
  (TransformerEngine PR 446), review thread on ``ck_to_aiter_mask_type``: no mask is 0; a
  window with left = -1 and right = 0 is causal, 1 when aligned top-left and 2 when aligned
  bottom-right; every other window is 3.  Causal includes the diagonal, so both window
  bounds are inclusive; the generic window (3) is aligned bottom-right like the causal
  bottom-right mask.  (Readings, not stated on the page.)
* Ragged (THD) batches -- "[ROCm] Fix THD/ragged dQ backward on the bf16 dq_shuffle path
  (gfx950)" (TransformerEngine PR 671), Verification: the reference there is block
  diagonal, i.e. every segment of a packed batch is an independent attention problem.
* Grouped-query attention -- same page, Tests: query heads share K/V heads in contiguous
  groups of Hq / Hkv (reading: head h uses K/V head h // (Hq // Hkv)).
* Additive bias -- "Update AITER subcommit and refactor internal AITER/CK FA API usage"
  (TransformerEngine PR 446), review threads on the bias strides: a bias of shape
  (bias_b, bias_h, Sq, Sk) with bias_b in {1, B} and bias_h in {1, H} (the shapes 11SS,
  1HSS, B1SS, BHSS; broadcast dimensions have stride 0), batch mode only; its gradient dbias
  has the shape of the bias and is the full (B, H, Sq, Sk) gradient summed over the
  broadcast dimensions.  Reading: the bias is added to the scaled logits before the mask
  and the softmax, so dbias = dS.
* Dropout -- same page, backward entry point: the random stream is a Philox generator
  driven by a seed and an offset.  Nothing else is stated; the readings taken: the
  generator is Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
  as 1, 2, 3", SC 2011); element (b, h, i, j) (segment/batch b, query head h, positions i, j
  inside the segment) uses byte (j mod 4) of output word (i mod 4) for key (seed low 32
  bits, seed high 32 bits) and counter (j div 4, i div 4, b*Hq + h, offset low 32 bits); it
  is kept iff that byte is < k = round((1 - p) * 256), and kept probabilities are scaled by
  256 / k.  Dropout acts on P in the P V product only (LSE is that of the full softmax), so
  dV = (P Z 256/k)^T dO, dP = (dO V^T) Z 256/k and dS = P (dP - D) with D = rowsum(dO O).
* Deterministic dQ accumulation -- "[CK_TILE] FMHA BWD Use Persistent Kernels in
  Deterministic Mode" (aiter PR 2216), Motivation and commit messages: dQ is accumulated as
  fp32 partials in an nsplits-deep workspace and converted back afterwards.  The order of
  the split sum is not stated; the reading taken is ascending split index.

For every (segment, query head h, K/V head g) with lengths Lq, Lk:

    S   = scale * Q_h K_g^T (+ bias[b, h])                   (Lq x Lk)
    (with dropout, P below is P Z 256/k in O = P V, dV and dP; Z the keep mask)
    LSE = log sum_{allowed j} exp(S_ij)       (-inf for a row with no allowed key)
    P   = exp(S - LSE) on allowed entries, 0 elsewhere
    O   = P V_g
    D_i = sum_c dO_ic O_ic
    dP  = dO V_g^T
    dS  = P * (dP - D 1^T)
    dQ_h = scale * dS K_g,   dK_g += scale * dS^T Q_h,   dV_g += P^T dO_h
    dbias[b, h] += dS   (summed over broadcast batch / head dimensions)

Layouts: batch mode arrays are [B, S, H, d] and LSE is [B, Hq, Sq]; group (THD) mode arrays
are [T, H, d] with ``seqstart`` offsets of length B+1 and LSE is [Hq, T].
"""

import numpy as np

MASK_NONE = 0
MASK_CAUSAL_TOP_LEFT = 1
MASK_CAUSAL_BOTTOM_RIGHT = 2
MASK_WINDOW = 3

_ROW_BLOCK = 512  # rows of S held at once (memory bound only; results do not depend on it)


def mask_geometry(mask_type, window_left, window_right, len_q, len_k):
    """Return (delta, left, right) such that key j is allowed for query i iff
    0 <= j < len_k, (left < 0 or j >= i + delta - left) and (right < 0 or j <= i + delta + right).

    Follows the mask-type table of the TransformerEngine PR 446 review thread
    (``ck_to_aiter_mask_type``): causal is the window (left=-1, right=0); top-left alignment
    puts the diagonal at j == i, bottom-right alignment at j == i + len_k - len_q.
    """
    if mask_type == MASK_NONE:
        return 0, -1, -1
    if mask_type == MASK_CAUSAL_TOP_LEFT:
        return 0, -1, 0
    if mask_type == MASK_CAUSAL_BOTTOM_RIGHT:
        return len_k - len_q, -1, 0
    if mask_type == MASK_WINDOW:
        return len_k - len_q, int(window_left), int(window_right)
    raise ValueError("unknown mask type %r" % (mask_type,))


def allowed(mask_type, window_left, window_right, len_q, len_k, rows=None, cols=None):
    """Boolean matrix allowed[i, j] for the given query rows and key columns."""
    delta, left, right = mask_geometry(mask_type, window_left, window_right, len_q, len_k)
    i = np.arange(len_q) if rows is None else np.asarray(rows)
    j = np.arange(len_k) if cols is None else np.asarray(cols)
    ii = i[:, None]
    jj = j[None, :]
    ok = (jj >= 0) & (jj < len_k) & (ii >= 0) & (ii < len_q)
    if left >= 0:
        ok = ok & (jj >= ii + delta - left)
    if right >= 0:
        ok = ok & (jj <= ii + delta + right)
    return ok


def _softmax_rows(s, ok):
    """Row softmax of s over the allowed entries; returns (P, LSE).  A row with no allowed
    entry has P = 0 and LSE = -inf."""
    if s.shape[1] == 0:  # no keys at all: every row is empty
        return np.zeros(s.shape), np.full(s.shape[0], -np.inf)
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 on disallowed entries
    z = e.sum(axis=1)
    z_safe = np.where(finite, z, 1.0)
    p = e / z_safe[:, None]
    lse = np.where(finite, m_safe + np.log(z_safe), -np.inf)
    return p, lse


def _segments(batch_mode, shape_q, shape_k, seqstart_q, seqstart_k):
    """Yield (b, q_rows, k_rows) where q_rows/k_rows index the leading axes of the arrays:
    (b, slice) in batch mode and slice in group mode."""
    if batch_mode:
        for b in range(shape_q[0]):
            yield b, (b, slice(0, shape_q[1])), (b, slice(0, shape_k[1]))
    else:
        nb = len(seqstart_q) - 1
        for b in range(nb):
            yield b, slice(int(seqstart_q[b]), int(seqstart_q[b + 1])), slice(
                int(seqstart_k[b]), int(seqstart_k[b + 1]))


def _bias_plane(bias, b, h):
    """The (Sq, Sk) plane of a (bias_b, bias_h, Sq, Sk) bias that batch b, head h reads."""
    return bias[b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0]


def _check_bias(bias, batch_mode, B, hq, sq, sk):
    if bias is None:
        return None
    if not batch_mode:
        raise ValueError("a bias needs batch mode")
    bias = np.asarray(bias, np.float64)
    if bias.ndim != 4 or bias.shape[0] not in (1, B) or bias.shape[1] not in (1, hq) or \
            bias.shape[2:] != (sq, sk):
        raise ValueError("bias must have shape (1|B, 1|Hq, Sq, Sk)")
    return bias


# ---------------------------------------------------------------------------------------
# Philox (Salmon et al., SC 2011): a counter-based generator.  N = 4 words of `bits` bits,
# two multipliers and two Weyl key increments; one round multiplies words 0 and 2 by the
# multipliers, and the output is (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
# lo(M0 c0)); the key grows by the Weyl constants between rounds.
# ---------------------------------------------------------------------------------------
PHILOX_4X32 = dict(bits=32, M=(0xD2511F53, 0xCD9E8D57), W=(0x9E3779B9, 0xBB67AE85))
PHILOX_4X64 = dict(bits=64, M=(0xD2E7470EE14C6C93, 0xCA5A826395121157),
                   W=(0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B))


def philox(counter, key, *, bits, M, W, rounds=10):
    """Philox-4x`bits`-`rounds` of a counter (4 arrays of words) under a key (2 words);
    returns the 4 output words.  Python integers, so arrays of any shape broadcast."""
    mask = (1 << bits) - 1
    c = [np.asarray(x, dtype=object) for x in counter]
    k0, k1 = int(key[0]), int(key[1])
    for r in range(rounds):
        if r:
            k0 = (k0 + W[0]) & mask
            k1 = (k1 + W[1]) & mask
        p0 = c[0] * M[0]
        p1 = c[2] * M[1]
        c = [(p1 >> bits) ^ c[1] ^ k0, p1 & mask, (p0 >> bits) ^ c[3] ^ k1, p0 & mask]
    return c


def dropout_threshold(p):
    """k = round((1 - p) * 256): bytes below k are kept; kept values are scaled by 256 / k."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    k = int(np.floor((1.0 - p) * 256.0 + 0.5))
    if k < 1:
        raise ValueError("dropout probability too close to 1")
    return k


def dropout_keep(seed, offset, b, h, hq, rows, cols, k):
    """Keep mask Z[i, j] of segment/batch b, query head h for the given positions."""
    ii = np.asarray(rows, dtype=np.int64)[:, None]
    jj = np.asarray(cols, dtype=np.int64)[None, :]
    ii, jj = np.broadcast_arrays(ii, jj)
    out = philox((jj >> 2, ii >> 2, np.full(ii.shape, b * hq + h, dtype=np.int64),
                  np.full(ii.shape, int(offset) & 0xFFFFFFFF, dtype=np.int64)),
                 (int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF), **PHILOX_4X32)
    words = np.stack([np.asarray(w, dtype=np.int64) for w in out])        # [4, ...]
    word = np.take_along_axis(words, (ii & 3)[None], axis=0)[0]
    byte = (word >> (8 * (jj & 3))) & 0xFF
    return byte < k


def _check_heads(hq, hkv):
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    return hq // hkv


def forward(q, k, v, *, scale, mask_type=MASK_NONE, window_left=-1, window_right=-1,
            seqstart_q=None, seqstart_k=None, bias=None, dropout=None):
    """Softmax attention forward in fp64.  Returns (O, LSE) in the layouts of the module
    docstring.  ``bias`` (batch mode): (1|B, 1|Hq, Sq, Sk), added to the scaled logits.
    ``dropout``: (p, seed, offset), see the module docstring."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    batch_mode = seqstart_q is None
    hq, hkv = q.shape[-2], k.shape[-2]
    group = _check_heads(hq, hkv)
    bias = _check_bias(bias, batch_mode, q.shape[0], hq, q.shape[1], k.shape[1]) if batch_mode \
        else _check_bias(bias, False, 0, hq, 0, 0)
    o = np.zeros(q.shape[:-1] + (v.shape[-1],), np.float64)
    if batch_mode:
        lse = np.full((q.shape[0], hq, q.shape[1]), -np.inf)
    else:
        lse = np.full((hq, q.shape[0]), -np.inf)
    for b, qs, ks in _segments(batch_mode, q.shape, k.shape, seqstart_q, seqstart_k):
        qb, kb, vb = q[qs], k[ks], v[ks]
        lq, lk = qb.shape[0], kb.shape[0]
        for h in range(hq):
            g = h // group
            for r0 in range(0, lq, _ROW_BLOCK):
                r1 = min(lq, r0 + _ROW_BLOCK)
                ok = allowed(mask_type, window_left, window_right, lq, lk, rows=np.arange(r0, r1))
                s = scale * (qb[r0:r1, h, :] @ kb[:, g, :].T)
                if bias is not None:
                    s = s + _bias_plane(bias, b, h)[r0:r1]
                p, l = _softmax_rows(s, ok)
                if dropout is not None:
                    p = p * _dropout_factor(dropout, b, h, hq, np.arange(r0, r1), lk)
                ob = p @ vb[:, g, :]
                if batch_mode:
                    o[b, r0:r1, h, :] = ob
                    lse[b, h, r0:r1] = l
                else:
                    o[qs][r0:r1, h, :] = ob
                    lse[h, qs.start + r0:qs.start + r1] = l
    return o, lse


def _dropout_factor(dropout, b, h, hq, rows, lk):
    """Z * 256/k for the given rows of segment b, head h (all lk keys)."""
    p_drop, seed, offset = dropout
    k = dropout_threshold(p_drop)
    return dropout_keep(seed, offset, b, h, hq, rows, np.arange(lk), k) * (256.0 / k)


def backward(q, k, v, do, *, scale, mask_type=MASK_NONE, window_left=-1, window_right=-1,
             seqstart_q=None, seqstart_k=None, bias=None, dropout=None):
    """Exact gradient of O = softmax(scale Q K^T + bias + mask) V in direction dO, fp64.

    Returns (dQ, dK, dV) shaped like (Q, K, V), and dbias (shaped like the bias) as a fourth
    element when a bias is given.  O, LSE and D are recomputed here from Q, K, V, so the
    result is the gradient of the exact forward."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    batch_mode = seqstart_q is None
    hq, hkv = q.shape[-2], k.shape[-2]
    group = _check_heads(hq, hkv)
    bias = _check_bias(bias, batch_mode, q.shape[0], hq, q.shape[1], k.shape[1]) if batch_mode \
        else _check_bias(bias, False, 0, hq, 0, 0)
    dbias = None if bias is None else np.zeros_like(bias)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b, qs, ks in _segments(batch_mode, q.shape, k.shape, seqstart_q, seqstart_k):
        qb, kb, vb, dob = q[qs], k[ks], v[ks], do[qs]
        lq, lk = qb.shape[0], kb.shape[0]
        dqb = np.zeros_like(qb)
        dkb = np.zeros_like(kb)
        dvb = np.zeros_like(vb)
        for h in range(hq):
            g = h // group
            for r0 in range(0, lq, _ROW_BLOCK):
                r1 = min(lq, r0 + _ROW_BLOCK)
                ok = allowed(mask_type, window_left, window_right, lq, lk, rows=np.arange(r0, r1))
                qh = qb[r0:r1, h, :]
                doh = dob[r0:r1, h, :]
                s = scale * (qh @ kb[:, g, :].T)
                if bias is not None:
                    s = s + _bias_plane(bias, b, h)[r0:r1]
                p, _ = _softmax_rows(s, ok)
                zf = 1.0 if dropout is None else _dropout_factor(dropout, b, h, hq, np.arange(r0, r1), lk)
                o = (p * zf) @ vb[:, g, :]
                d = (doh * o).sum(axis=1)
                dp = (doh @ vb[:, g, :].T) * zf
                ds = p * (dp - d[:, None])
                if dbias is not None:
                    _bias_plane(dbias, b, h)[r0:r1] += ds
                dqb[r0:r1, h, :] = scale * (ds @ kb[:, g, :])
                dkb[:, g, :] += scale * (ds.T @ qh)
                dvb[:, g, :] += (p * zf).T @ doh
        dq[qs] = dqb
        dk[ks] = dkb
        dv[ks] = dvb
    if dbias is not None:
        return dq, dk, dv, dbias
    return dq, dk, dv


# ---------------------------------------------------------------------------------------
# Row-sampled forms of the same definition, for inputs too large for the full oracle.
# They evaluate single output rows of dQ (one query row) or of dK/dV (one key row) from the
# same formulas; ``tests/test_oracle.py`` pins them to ``backward`` on small inputs.
# ---------------------------------------------------------------------------------------

def _segment_arrays(x, batch_mode, b, seqstart):
    if batch_mode:
        return x[b]
    return x[int(seqstart[b]):int(seqstart[b + 1])]


def row_statistics(q, k, v, do, *, scale, segment, heads, mask_type=MASK_NONE,
                   window_left=-1, window_right=-1, seqstart_q=None, seqstart_k=None):
    """For one segment and the given query heads, return dict h -> (LSE[Lq], D[Lq]) where
    D_i = sum_c dO_ic O_ic with O the exact fp64 forward output."""
    batch_mode = seqstart_q is None
    group = _check_heads(q.shape[-2], k.shape[-2])
    qb = np.asarray(_segment_arrays(q, batch_mode, segment, seqstart_q), np.float64)
    kb = np.asarray(_segment_arrays(k, batch_mode, segment, seqstart_k), np.float64)
    vb = np.asarray(_segment_arrays(v, batch_mode, segment, seqstart_k), np.float64)
    dob = np.asarray(_segment_arrays(do, batch_mode, segment, seqstart_q), np.float64)
    lq, lk = qb.shape[0], kb.shape[0]
    out = {}
    for h in heads:
        g = h // group
        lse = np.full(lq, -np.inf)
        dd = np.zeros(lq)
        for r0 in range(0, lq, _ROW_BLOCK):
            r1 = min(lq, r0 + _ROW_BLOCK)
            ok = allowed(mask_type, window_left, window_right, lq, lk, rows=np.arange(r0, r1))
            s = scale * (qb[r0:r1, h, :] @ kb[:, g, :].T)
            p, l = _softmax_rows(s, ok)
            o = p @ vb[:, g, :]
            lse[r0:r1] = l
            dd[r0:r1] = (dob[r0:r1, h, :] * o).sum(axis=1)
        out[h] = (lse, dd)
    return out


def dq_rows(q, k, v, do, *, scale, segment, head, rows, stats, mask_type=MASK_NONE,
            window_left=-1, window_right=-1, seqstart_q=None, seqstart_k=None):
    """dQ for the given query rows (segment-local indices) of one query head.  ``stats`` is
    the (LSE, D) pair of that head from ``row_statistics``."""
    batch_mode = seqstart_q is None
    group = _check_heads(q.shape[-2], k.shape[-2])
    g = head // group
    qb = np.asarray(_segment_arrays(q, batch_mode, segment, seqstart_q), np.float64)
    kb = np.asarray(_segment_arrays(k, batch_mode, segment, seqstart_k), np.float64)
    vb = np.asarray(_segment_arrays(v, batch_mode, segment, seqstart_k), np.float64)
    dob = np.asarray(_segment_arrays(do, batch_mode, segment, seqstart_q), np.float64)
    lq, lk = qb.shape[0], kb.shape[0]
    rows = np.asarray(rows)
    lse, dd = stats
    ok = allowed(mask_type, window_left, window_right, lq, lk, rows=rows)
    s = scale * (qb[rows, head, :] @ kb[:, g, :].T)
    lse_r = lse[rows]
    fin = np.isfinite(lse_r)
    p = np.where(ok, np.exp(s - np.where(fin, lse_r, 0.0)[:, None]), 0.0)
    dp = dob[rows, head, :] @ vb[:, g, :].T
    ds = p * (dp - dd[rows][:, None])
    return scale * (ds @ kb[:, g, :])


def dkdv_rows(q, k, v, do, *, scale, segment, kv_head, rows, stats, mask_type=MASK_NONE,
              window_left=-1, window_right=-1, seqstart_q=None, seqstart_k=None):
    """dK and dV for the given key rows (segment-local) of one K/V head, summed over the query
    heads of its group.  ``stats`` maps each of those query heads to its (LSE, D)."""
    batch_mode = seqstart_q is None
    group = _check_heads(q.shape[-2], k.shape[-2])
    qb = np.asarray(_segment_arrays(q, batch_mode, segment, seqstart_q), np.float64)
    kb = np.asarray(_segment_arrays(k, batch_mode, segment, seqstart_k), np.float64)
    vb = np.asarray(_segment_arrays(v, batch_mode, segment, seqstart_k), np.float64)
    dob = np.asarray(_segment_arrays(do, batch_mode, segment, seqstart_q), np.float64)
    lq, lk = qb.shape[0], kb.shape[0]
    rows = np.asarray(rows)
    dk = np.zeros((len(rows), kb.shape[-1]))
    dv = np.zeros((len(rows), vb.shape[-1]))
    for h in range(kv_head * group, (kv_head + 1) * group):
        lse, dd = stats[h]
        ok = allowed(mask_type, window_left, window_right, lq, lk, cols=rows)  # [Lq, n]
        s = scale * (qb[:, h, :] @ kb[rows, kv_head, :].T)
        fin = np.isfinite(lse)
        p = np.where(ok, np.exp(s - np.where(fin, lse, 0.0)[:, None]), 0.0)
        dp = dob[:, h, :] @ vb[rows, kv_head, :].T
        ds = p * (dp - dd[:, None])
        dk += scale * (ds.T @ qb[:, h, :])
        dv += p.T @ dob[:, h, :]
    return dk, dv


def rowsum_product(a, b):
    """D_i = sum_c a_ic b_ic in fp64 over the last axis (D = rowsum(dO * O) for the given O)."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64)).sum(axis=-1)


# ---------------------------------------------------------------------------------------
# Deterministic split reduction (aiter PR 2216, Motivation: dQ is "split, stored, and
# converted back"; TransformerEngine PR 671, Root cause: the fp32 convert post-kernel).
# ---------------------------------------------------------------------------------------

def _bf16_round_bits(x32):
    """Round float32 values to bfloat16 with round-to-nearest, ties to even; returns uint16
    bit patterns.  (NaN is not produced by the path and is not handled specially.)"""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def dq_split_reduce(partials, scale):
    """dQ = bf16_RNE(fp32(scale) * sum_s partials[s]), the fp32 sum taken one split at a time
    in ascending split index.  ``partials`` is float32 [nsplits, ...]; returns uint16 bf16
    bit patterns of shape partials.shape[1:].  An empty split list gives +0."""
    partials = np.asarray(partials, np.float32)
    acc = np.zeros(partials.shape[1:], np.float32)
    for s in range(partials.shape[0]):
        acc = (acc + partials[s]).astype(np.float32)
    out = (acc * np.float32(scale)).astype(np.float32)
    return _bf16_round_bits(out)
