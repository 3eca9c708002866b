"""Python binding of the C-ABI library: argument marshalling only.

PyTorch provides device memory (the chunk pool, the workspace, q/out) and the
current stream; every step of the decode path runs in the library's HIP
kernels.
"""

from __future__ import annotations

import ctypes
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import _capi
from ._capi import CaError, check, load

HEAD_DIM = 128
CHUNK = 64


def slot_bytes(heads: int, head_dim: int = HEAD_DIM, chunk: int = CHUNK) -> int:
    return int(load().ca_slot_bytes(heads, head_dim, chunk))


_copy_path_warm = False


def _warm_copy_path(torch, dev_buf) -> None:
    """Make one pinned host-to-device copy of more than 16 KiB, once per
    process.  The HIP runtime sets up its path for such copies at the first
    one (about 6 ms on MI355X, most of it CPU time; later copies take a few
    microseconds), and a table upload that is the first would pay it inside a
    decode step."""
    global _copy_path_warm
    n = min(dev_buf.numel(), 64 << 10)
    if _copy_path_warm or n <= 16 << 10:
        return
    src = torch.zeros(n, dtype=torch.uint8, pin_memory=True)
    dev_buf[:n].copy_(src, non_blocking=True)
    torch.cuda.current_stream(dev_buf.device).synchronize()
    _copy_path_warm = True


def _tokens(tokens) -> np.ndarray:
    if type(tokens) is np.ndarray and tokens.dtype == np.int32 and tokens.ndim == 1 and tokens.flags.c_contiguous:
        return tokens
    return np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))


def _ptr_i32(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class ChunkAttention:
    """Prefix-tree KV cache plus the two-phase decode-step attention.

    heads: head count; capacity_slots: pool size in 64-token chunk slots.
    device: a torch device for the pool, or None for a host-only context
    (tree and tables only; attend is unavailable).  share=False builds the
    unshared paged layout (every sequence keeps its own chunks);
    two_phase=False keeps the shared layout but runs no chunk-first phase
    (every sequence streams its whole path).
    """

    def __init__(self, heads: int, capacity_slots: int, device="cuda", share: bool = True,
                 head_dim: int = HEAD_DIM, chunk_size: int = CHUNK, two_phase: bool = True):
        self.lib = load()
        self.heads, self.head_dim, self.chunk = heads, head_dim, chunk_size
        ctx = ctypes.c_void_p()
        flags = (0 if share else _capi.CA_CREATE_UNSHARED) | (0 if two_phase else _capi.CA_CREATE_NO_CHUNK_FIRST)
        rc = self.lib.ca_create_ex(heads, head_dim, chunk_size, flags, ctypes.byref(ctx))
        if rc != 0:
            raise CaError(rc, "ca_create_ex failed")
        self.ctx = ctx
        self.device = device
        self.pool = None
        self.ws = None
        self.stage = None
        self._n_live = 0
        if device is None:
            check(self.ctx, self.lib.ca_attach_pool(self.ctx, None, capacity_slots))
        else:
            import torch
            nbytes = capacity_slots * slot_bytes(heads, head_dim, chunk_size)
            self.pool = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            # before the pool is attached, while its contents mean nothing
            _warm_copy_path(torch, self.pool)
            # what the per-step argument checks use, looked up once
            self._torch, self._f16 = torch, torch.float16
            raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
            index = self.pool.device.index
            self._current_stream = (lambda: raw(index)) if raw is not None else (
                lambda: torch.cuda.current_stream(index).cuda_stream)
            check(self.ctx, self.lib.ca_attach_pool(self.ctx, ctypes.c_void_p(self.pool.data_ptr()),
                                                   capacity_slots))
            self._lend_staging(3 << 16)

    # -- lifetime -------------------------------------------------------------
    def close(self):
        if getattr(self, "ctx", None):
            self.lib.ca_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- helpers --------------------------------------------------------------
    def _stream(self, stream=None):
        """The hipStream_t of `stream`, else of the pool device's current stream."""
        if self.device is None:
            return None
        return stream.cuda_stream if stream is not None else self._current_stream()

    def _f16_ptr(self, name: str, x, shape):
        """Device address of a contiguous fp16 CUDA tensor of the given shape."""
        try:
            if x.dtype is self._f16 and x.is_cuda and x.shape == shape and x.is_contiguous():
                return x.data_ptr()
        except AttributeError:
            pass
        if not isinstance(x, self._torch.Tensor) or x.dtype != self._f16 or not x.is_cuda:
            raise TypeError(f"{name} must be a float16 CUDA tensor")
        raise ValueError(f"{name} must be contiguous {list(shape)}")

    def _kv(self, k, v, n: int):
        if self.device is None:
            if k is not None or v is not None:
                raise ValueError("a host-only context takes no K/V")
            return None, None
        shape = (n, self.heads, self.head_dim)
        return self._f16_ptr("k", k, shape), self._f16_ptr("v", v, shape)

    # -- tree -----------------------------------------------------------------
    def insert(self, seq_id: int, tokens, k=None, v=None, stream=None) -> int:
        t = _tokens(tokens)
        kp, vp = self._kv(k, v, len(t)) if len(t) else (None, None)
        matched = ctypes.c_int32(0)
        check(self.ctx, self.lib.ca_insert(self.ctx, seq_id, _ptr_i32(t), len(t), kp, vp, self._stream(stream),
                                           ctypes.byref(matched)))
        self._n_live += 1
        return matched.value

    def append(self, seq_id: int, tokens, k=None, v=None, stream=None) -> None:
        t = _tokens(tokens)
        kp, vp = self._kv(k, v, len(t)) if len(t) else (None, None)
        check(self.ctx, self.lib.ca_append(self.ctx, seq_id, _ptr_i32(t), len(t), kp, vp, self._stream(stream)))

    def append_batch(self, seq_ids, tokens, k=None, v=None, stream=None) -> None:
        """One token per sequence: tokens[j] with K/V row j goes to seq_ids[j]."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64).reshape(-1))
        t = _tokens(tokens)
        if len(ids) != len(t):
            raise ValueError("one token per sequence id")
        kp, vp = self._kv(k, v, len(t)) if len(t) else (None, None)
        check(self.ctx, self.lib.ca_append_batch(self.ctx, len(ids),
                                                 ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                                 _ptr_i32(t), kp, vp, self._stream(stream)))

    def remove(self, seq_id: int) -> None:
        check(self.ctx, self.lib.ca_remove(self.ctx, seq_id))
        self._n_live -= 1

    def sequences(self) -> List[int]:
        n = check(self.ctx, self.lib.ca_list_sequences(self.ctx, None, 0))
        buf = (ctypes.c_int64 * max(n, 1))()
        check(self.ctx, self.lib.ca_list_sequences(self.ctx, buf, n))
        return [int(buf[i]) for i in range(n)]

    def set_option(self, option: int, value: int) -> None:
        check(self.ctx, self.lib.ca_set_option(self.ctx, option, value))

    def export_table(self) -> Tuple[np.ndarray, List[int]]:
        nr, ns = ctypes.c_int(0), ctypes.c_int(0)
        check(self.ctx, self.lib.ca_export_table(self.ctx, None, 0, None, 0, ctypes.byref(nr), ctypes.byref(ns)))
        rows = np.zeros((max(nr.value, 1), 7), np.int32)
        order = np.zeros(max(ns.value, 1), np.int64)
        check(self.ctx, self.lib.ca_export_table(
            self.ctx, rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), nr.value,
            order.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ns.value, ctypes.byref(nr), ctypes.byref(ns)))
        return rows[: nr.value], [int(x) for x in order[: ns.value]]

    def export_plan(self) -> bytes:
        """The device table image of the current plan (for bit-exact comparisons)."""
        n = ctypes.c_size_t(0)
        check(self.ctx, self.lib.ca_export_plan(self.ctx, None, 0, ctypes.byref(n)))
        buf = ctypes.create_string_buffer(max(n.value, 1))
        check(self.ctx, self.lib.ca_export_plan(self.ctx, buf, n.value, ctypes.byref(n)))
        return buf.raw[: n.value]

    def stats(self) -> Dict[str, float]:
        s = _capi.ca_stats_t()
        check(self.ctx, self.lib.ca_stats(self.ctx, ctypes.byref(s)))
        return {name: getattr(s, name) for name, _ in s._fields_}

    def workspace_bytes(self) -> int:
        n = ctypes.c_size_t(0)
        check(self.ctx, self.lib.ca_workspace_bytes(self.ctx, ctypes.byref(n)))
        return int(n.value)

    def staging_bytes(self) -> int:
        n = ctypes.c_size_t(0)
        check(self.ctx, self.lib.ca_staging_bytes(self.ctx, ctypes.byref(n)))
        return int(n.value)

    def _lend_staging(self, nbytes: int) -> None:
        """Pinned host memory (a torch tensor) for the table uploads, cut to a
        256-byte aligned start."""
        import torch
        buf = torch.empty(nbytes + 256, dtype=torch.uint8, pin_memory=True)
        off = (-buf.data_ptr()) % 256
        view = buf[off:off + nbytes]
        check(self.ctx, self.lib.ca_attach_staging(self.ctx, ctypes.c_void_p(view.data_ptr()), nbytes))
        self.stage = view  # the view keeps the whole buffer alive

    # -- step -----------------------------------------------------------------
    def ensure_workspace(self) -> None:
        import torch
        need = self.workspace_bytes()
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(need + need // 4, 4096), dtype=torch.uint8, device=self.pool.device)
            check(self.ctx, self.lib.ca_attach_workspace(self.ctx, ctypes.c_void_p(self.ws.data_ptr()),
                                                         self.ws.numel()))
        stage = self.staging_bytes()
        if self.stage is None or self.stage.numel() < stage:
            self._lend_staging(max(stage + stage // 4, 3 << 16))

    def _qo(self, q, out):
        """q and out (made like q when None) checked; returns out and both addresses."""
        shape = (self._n_live, self.heads, self.head_dim)
        qp = self._f16_ptr("q (rows in ascending seq id)", q, shape)
        if out is None:
            out = self._torch.empty_like(q)
        else:
            try:
                ok = out.dtype is self._f16 and out.shape == shape and out.is_contiguous()
            except AttributeError:
                ok = False
            if not ok:
                raise ValueError("out must match q")
        return out, qp, out.data_ptr()

    def attend(self, q, out=None, stream=None):
        """out[r] = softmax(q[r] K_r^T / sqrt(d)) V_r for the r-th live sequence."""
        if self.device is None:
            raise CaError(-9, "host-only context")
        out, qp, op = self._qo(q, out)
        args = (self.ctx, qp, op, self._stream(stream))
        rc = self.lib.ca_attend(*args)
        if rc == -7:
            # the tree outgrew the workspace (nothing was launched): grow it
            self.ensure_workspace()
            rc = self.lib.ca_attend(*args)
        check(self.ctx, rc)
        return out

    def attend_noalloc(self, q, out, stream=None):
        """attend() with the step's workspace in the library's static device
        scratch (ca_attend_noalloc): no allocation by the library or here;
        out must be given."""
        if self.device is None:
            raise CaError(-9, "host-only context")
        if out is None:
            raise ValueError("attend_noalloc writes into a caller-provided out")
        out, qp, op = self._qo(q, out)
        check(self.ctx, self.lib.ca_attend_noalloc(self.ctx, qp, op, self._stream(stream)))
        return out

    def decode_step(self, tokens, k, v, q, out=None, stream=None):
        """Append tokens[r] with K/V row r to the r-th live sequence (ascending
        id), then attend with q; returns out (ca_decode_step)."""
        if self.device is None:
            raise CaError(-9, "host-only context")
        t = _tokens(tokens)
        if len(t) != self._n_live:
            raise ValueError("one token per live sequence")
        kp, vp = self._kv(k, v, len(t))
        out, qp, op = self._qo(q, out)
        rc = self.lib.ca_decode_step(self.ctx, t.ctypes.data, kp, vp, qp, op, self._stream(stream))
        if rc == -7:
            # the tokens are stored; the tree outgrew the workspace: grow it
            # and run the step's attention
            self.ensure_workspace()
            return self.attend(q, out, stream)
        check(self.ctx, rc)
        return out

    def prepare(self, stream=None) -> None:
        self.ensure_workspace()
        check(self.ctx, self.lib.ca_prepare(self.ctx, self._stream(stream)))

    def attend_phase(self, phase: int, q, out, stream=None) -> None:
        check(self.ctx, self.lib.ca_attend_phase(self.ctx, phase, ctypes.c_void_p(q.data_ptr()),
                                                 ctypes.c_void_p(out.data_ptr()), self._stream(stream)))


def load_workload(ca: ChunkAttention, wl, device="cuda", stream=None, segments: Optional[dict] = None) -> None:
    """Insert every sequence of a seeded workload (ids 0..N-1) with its K/V.

    A workload built from segments has each segment's K/V copied to the device
    once (kept in ``segments`` when given, so several contexts can share the
    copies) and every sequence's K/V assembled on the device; other workloads
    copy each sequence's rows."""
    import torch
    segs = getattr(wl, "segments", None)
    if segs is None:
        for i in range(wl.n_seq):
            k, v = wl.seq_kv(i)
            kt = torch.from_numpy(np.ascontiguousarray(k)).to(device)
            vt = torch.from_numpy(np.ascontiguousarray(v)).to(device)
            ca.insert(i, wl.seq_tokens(i), kt, vt, stream=stream)
        return
    cache = segments if segments is not None else {}
    for i in range(wl.n_seq):
        for j in wl.paths[i]:
            if j not in cache:
                cache[j] = (torch.from_numpy(segs[j].k).to(device), torch.from_numpy(segs[j].v).to(device))
        parts = [cache[j] for j in wl.paths[i]]
        kt = torch.cat([p[0] for p in parts]) if len(parts) > 1 else parts[0][0]
        vt = torch.cat([p[1] for p in parts]) if len(parts) > 1 else parts[0][1]
        ca.insert(i, wl.seq_tokens(i), kt, vt, stream=stream)
        if len(parts) > 1 and stream is not None:
            # the copies read kt/vt on another stream than torch's: keep them
            # alive until that stream is past them
            stream.synchronize()


def slots_needed(wl, chunk: int = CHUNK, share: bool = True) -> int:
    """Upper bound of the slots a workload occupies (splits included)."""
    if not share:
        return int(sum((int(n) + chunk - 1) // chunk for n in wl.lengths()))
    segs = getattr(wl, "segments", None)
    if segs is not None and all(s.length % chunk == 0 for p in wl.paths for s in
                                (segs[j] for j in p[:-1])):
        # segment boundaries on chunk boundaries: one chunk run per segment
        used = sorted({j for p in wl.paths for j in p})
        return int(sum((segs[j].length + chunk - 1) // chunk for j in used))
    # every sequence at most adds its own chunks plus one split
    return int(sum((int(n) + chunk - 1) // chunk + 1 for n in wl.lengths()))
