"""fp64 reference attention for one decode step.  TEST INFRASTRUCTURE ONLY.

What is computed (ChunkAttention explainer, 0h-n0.github.io/posts/paper-2402-15220,
sections "Phase 1" / "Phase 2" formulas and the "Algorithm" sketch; paperlayer.ai
summary of arXiv 2402.15220v4, section 2.2):

    For each live sequence i (one query token per sequence in iteration-based
    batching, attention independent per sequence) and each head h,
        x_j   = (q_ih . k_ijh) / sqrt(d)                 over all stored tokens j
        out_ih = sum_j softmax(x)_j v_ijh

Everything is done in float64 after an exact upcast of the float16 inputs.
The two-phase partition of the method is an exact re-association of this sum;
``partial`` and ``merge`` below state that re-association (explainer, "output
combination" formula and the code of the sketch: per part a running max m,
an unnormalised sum s of exp(x - m) and an unnormalised output o).
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence, Tuple

import numpy as np

Partial = Tuple[np.ndarray, np.ndarray, np.ndarray]  # (o [H,d], m [H], s [H])


def default_scale(head_dim: int) -> float:
    """1/sqrt(d_k), as in the explainer's formulas."""
    return 1.0 / math.sqrt(head_dim)


def attend_sequence(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    scale: float | None = None) -> np.ndarray:
    """softmax(q K^T * scale) V for one sequence.

    q: [H, d]; k, v: [L, H, d] (any float dtype, upcast exactly to fp64).
    Returns float64 [H, d].  L must be >= 1.
    """
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    if k64.shape[0] < 1:
        raise ValueError("a sequence needs at least one stored token")
    if scale is None:
        scale = default_scale(q64.shape[-1])
    kh = np.ascontiguousarray(k64.transpose(1, 0, 2))  # [H, L, d]
    vh = np.ascontiguousarray(v64.transpose(1, 0, 2))
    x = np.matmul(kh, q64[:, :, None])[:, :, 0] * scale  # [H, L]
    x = x - x.max(axis=1, keepdims=True)
    w = np.exp(x)
    w = w / w.sum(axis=1, keepdims=True)
    return np.matmul(w[:, None, :], vh)[:, 0, :]


def decode_step(q: np.ndarray, seq_kv: Iterable[Tuple[np.ndarray, np.ndarray]],
                scale: float | None = None) -> np.ndarray:
    """One decode step: row i of q attends over the i-th (K, V) pair.

    q: [N, H, d]; seq_kv yields N pairs of [L_i, H, d].  Returns fp64 [N, H, d].
    """
    outs = []
    for i, (k, v) in enumerate(seq_kv):
        outs.append(attend_sequence(q[i], k, v, scale))
    return np.stack(outs) if outs else np.zeros((0,) + q.shape[1:], np.float64)


def decode_workload(wl, rows: Sequence[int] | None = None,
                    scale: float | None = None) -> np.ndarray:
    """decode_step over a workload object (``workloads``); optionally a row subset."""
    rows = list(range(wl.n_seq)) if rows is None else list(rows)
    out = np.empty((len(rows), wl.heads, wl.head_dim), np.float64)
    for n, i in enumerate(rows):
        k, v = wl.seq_kv(i)
        out[n] = attend_sequence(wl.q[i], k, v, scale)
    return out


# --- the partial-result form used by the two-phase partition -----------------

def partial(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None) -> Partial:
    """Attention of q over one part of the keys, unnormalised.

    Returns (o, m, s) with m = max_j x_j, s = sum_j exp(x_j - m),
    o = sum_j exp(x_j - m) v_j, per head.  An empty part is the identity
    element (o = 0, m = -inf, s = 0).
    """
    q64 = np.asarray(q, dtype=np.float64)
    H, d = q64.shape
    if scale is None:
        scale = default_scale(d)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    if k64.shape[0] == 0:
        return np.zeros((H, d)), np.full(H, -np.inf), np.zeros(H)
    kh = np.ascontiguousarray(k64.transpose(1, 0, 2))
    vh = np.ascontiguousarray(v64.transpose(1, 0, 2))
    x = np.matmul(kh, q64[:, :, None])[:, :, 0] * scale
    m = x.max(axis=1)
    e = np.exp(x - m[:, None])
    return np.matmul(e[:, None, :], vh)[:, 0, :], m, e.sum(axis=1)


def merge(a: Partial, b: Partial) -> Partial:
    """Combine two partials: M = max(m_a, m_b), weights exp(m - M)."""
    oa, ma, sa = a
    ob, mb, sb = b
    M = np.maximum(ma, mb)
    # exp(-inf - finite) = 0; both -inf only for two empty parts -> stay empty.
    with np.errstate(invalid="ignore"):
        wa = np.where(np.isneginf(ma), 0.0, np.exp(ma - M))
        wb = np.where(np.isneginf(mb), 0.0, np.exp(mb - M))
    return wa[:, None] * oa + wb[:, None] * ob, M, wa * sa + wb * sb


def merge_all(parts: Sequence[Partial]) -> Partial:
    acc = parts[0]
    for p in parts[1:]:
        acc = merge(acc, p)
    return acc


def finalize(p: Partial) -> np.ndarray:
    o, _, s = p
    return o / s[:, None]


def two_phase(q: np.ndarray, k_prefix: np.ndarray, v_prefix: np.ndarray,
              k_suffix: np.ndarray, v_suffix: np.ndarray,
              scale: float | None = None) -> np.ndarray:
    """The explainer's combination of a prefix part and a suffix part:
    O = (e^{m_p} O_p + e^{m_s} O_s) / (e^{m_p} + e^{m_s}) with normalised parts
    and m the log-sum-exp of each part, written here directly in that form."""
    op, mp, sp = partial(q, k_prefix, v_prefix, scale)
    os_, ms, ss = partial(q, k_suffix, v_suffix, scale)
    lse_p = mp + np.log(sp)
    lse_s = ms + np.log(ss)
    Op = op / sp[:, None]
    Os = os_ / ss[:, None]
    top = np.maximum(lse_p, lse_s)
    wp = np.exp(lse_p - top)
    ws = np.exp(lse_s - top)
    return (wp[:, None] * Op + ws[:, None] * Os) / (wp + ws)[:, None]


def allclose_report(got: np.ndarray, ref: np.ndarray, atol: float = 2e-3, rtol: float = 1e-2) -> dict:
    """Elementwise |got - ref| <= atol + rtol*|ref|, plus rel-L2 and max error."""
    got64 = np.asarray(got, dtype=np.float64)
    ref64 = np.asarray(ref, dtype=np.float64)
    err = np.abs(got64 - ref64)
    bad = err > atol + rtol * np.abs(ref64)
    return {
        "ok": bool(not bad.any() and np.isfinite(got64).all()),
        "n_bad": int(bad.sum()),
        "max_abs": float(err.max()) if err.size else 0.0,
        "rel_l2": float(np.linalg.norm(got64 - ref64) / max(np.linalg.norm(ref64), 1e-300)),
    }
