"""Python binding of libbeamstep.so (the C ABI in include/beamstep.h).

Argument marshalling only: every step of the beam search runs in the HIP
kernels of the library. torch tensors supply device memory and the HIP stream
(``data_ptr()`` and ``torch.cuda.current_stream().cuda_stream``). The library
must have been built (``__graft_entry__.build()``); importing the binding
without it raises, and there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbeamstep.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "beamstep.h")

BS_OK, BS_EINVAL, BS_ENOMEM, BS_EDEVICE, BS_ESTATE = 0, -1, -2, -3, -4
BS_F32, BS_BF16 = 0, 1
BS_LP_NONE, BS_LP_GNMT, BS_LP_POW = 0, 1, 2
BS_STOP_TRUE, BS_STOP_HEURISTIC, BS_STOP_NEVER = 0, 1, 2
BS_PRUNE_TOPW, BS_PRUNE_TOP2W = 0, 1
BS_SELECT_FUSED, BS_SELECT_TWO_PASS = 0, 1

DTYPES = {"f32": BS_F32, "bf16": BS_BF16}
# torch dtypes that hold each logits type (bf16 may come as its 16-bit pattern)
LOGIT_DTYPES = {"f32": {"float32"}, "bf16": {"bfloat16", "int16", "uint16"}}
LPS = {"none": BS_LP_NONE, "gnmt": BS_LP_GNMT, "pow": BS_LP_POW}
STOPS = {"true": BS_STOP_TRUE, "heuristic": BS_STOP_HEURISTIC, "never": BS_STOP_NEVER}
PRUNES = {"topw": BS_PRUNE_TOPW, "top2w": BS_PRUNE_TOP2W}
SELECTS = {"fused": BS_SELECT_FUSED, "two_pass": BS_SELECT_TWO_PASS}


class bs_config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("beam", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("max_steps", ctypes.c_int32), ("eos_id", ctypes.c_int32), ("pad_id", ctypes.c_int32),
        ("logits_dtype", ctypes.c_int32), ("lp", ctypes.c_int32), ("alpha", ctypes.c_double),
        ("stop", ctypes.c_int32), ("num_return", ctypes.c_int32), ("tile_elems", ctypes.c_int32),
        ("prune", ctypes.c_int32), ("select", ctypes.c_int32),
    ]


class bs_kv_desc(ctypes.Structure):
    _fields_ = [
        ("n_planes", ctypes.c_int32), ("planes", ctypes.POINTER(ctypes.c_void_p)),
        ("row_stride", ctypes.c_int64), ("pos_stride", ctypes.c_int64),
        ("pos_offset", ctypes.c_int64), ("bytes_per_pos", ctypes.c_int64),
    ]


class bs_kv_pool(ctypes.Structure):
    _fields_ = [
        ("n_planes", ctypes.c_int32), ("pools", ctypes.POINTER(ctypes.c_void_p)),
        ("block_stride", ctypes.c_int64), ("pos_stride", ctypes.c_int64),
        ("bytes_per_pos", ctypes.c_int64),
    ]


class BeamStepError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {bs_strerror(status)} ({status})")


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libbeamstep.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.bs_strerror.restype = ctypes.c_char_p
        L.bs_strerror.argtypes = [ctypes.c_int]
        L.bs_create.argtypes = [ctypes.POINTER(bs_config), P, ctypes.POINTER(P)]
        L.bs_reset.argtypes = [P]
        L.bs_step.argtypes = [P, P, i64, P, P, P, P]
        L.bs_reorder_kv.argtypes = [P, ctypes.POINTER(bs_kv_desc), i32]
        L.bs_reorder_kv_timed.argtypes = [P, ctypes.POINTER(bs_kv_desc), i32, P, P]
        L.bs_finalize.argtypes = [P, P, P, P]
        L.bs_last_selection.argtypes = [P, P, P]
        L.bs_get_finished.argtypes = [P, P, P, P, P, P, P]
        L.bs_steps_taken.argtypes = [P]
        L.bs_state_size.argtypes = [P, ctypes.POINTER(i64)]
        L.bs_state_save.argtypes = [P, P, i64]
        L.bs_state_load.argtypes = [P, P, i64]
        L.bs_destroy.argtypes = [P]
        L.bs_destroy.restype = None
        L.bs_kv_paged_create.argtypes = [P, i32, i32, ctypes.POINTER(P)]
        L.bs_kv_paged_reset.argtypes = [P]
        L.bs_kv_paged_table.argtypes = [P, ctypes.POINTER(P), ctypes.POINTER(i32)]
        L.bs_kv_paged_reorder.argtypes = [P, ctypes.POINTER(bs_kv_pool), i32]
        L.bs_kv_paged_status.argtypes = [P, P, P]
        L.bs_kv_paged_destroy.argtypes = [P]
        L.bs_kv_paged_destroy.restype = None
        L.bs_verify_create.argtypes = [i32, i32, i32, i32, P, ctypes.POINTER(P)]
        L.bs_verify.argtypes = [P, P, i64, P, P, P]
        L.bs_verify_ex.argtypes = [P, P, i64, P, i32, i32, P, P, P]
        L.bs_verify_noalloc.argtypes = [P, P, i32, i32, i32, i32, i64, P, P, P]
        L.bs_verify_destroy.argtypes = [P]
        L.bs_verify_destroy.restype = None
        for name in ("bs_create", "bs_reset", "bs_step", "bs_reorder_kv", "bs_reorder_kv_timed",
                     "bs_finalize",
                     "bs_last_selection", "bs_get_finished", "bs_steps_taken",
                     "bs_state_size", "bs_state_save", "bs_state_load",
                     "bs_kv_paged_create", "bs_kv_paged_reset", "bs_kv_paged_table",
                     "bs_kv_paged_reorder", "bs_kv_paged_status",
                     "bs_verify_create", "bs_verify", "bs_verify_ex", "bs_verify_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def declared_functions() -> list:
    """Names of the functions include/beamstep.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bs_[a-z_]+)\s*\(", text)))


def _check(status: int, call: str) -> None:
    if status != BS_OK:
        raise BeamStepError(status, call)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _rows(t, what: str, rows: int = 0, cols: int = 0, dtypes=None, need_gpu: bool = True) -> int:
    """Row stride, in elements, of a tensor of rows [rows, n] or [a, b, n]
    (row r at r * stride), after checking that it can hold what a kernel
    will read or write: at least ``rows`` rows of ``cols`` contiguous
    elements, evenly spaced, of one of ``dtypes``, on the GPU. The library
    takes plain pointers and cannot check sizes itself."""
    if need_gpu and not t.is_cuda:
        raise ValueError(f"{what}: a GPU tensor is needed")
    if dtypes and str(t.dtype).replace("torch.", "") not in dtypes:
        raise ValueError(f"{what}: dtype {t.dtype}, expected one of {sorted(dtypes)}")
    if t.dim() not in (2, 3) or t.stride(-1) != 1:
        raise ValueError(f"{what}: rows of contiguous elements expected, [rows, n] or [a, b, n]")
    if t.dim() == 3 and t.shape[0] > 1 and t.shape[1] > 1 and t.stride(0) != t.shape[1] * t.stride(1):
        raise ValueError(f"{what}: rows of [a, b, n] must be evenly spaced")
    n = t.shape[0] if t.dim() == 2 else t.shape[0] * t.shape[1]
    if n < rows:
        raise ValueError(f"{what}: {n} rows, {rows} needed")
    if t.shape[-1] < cols:
        raise ValueError(f"{what}: rows of {t.shape[-1]} elements, {cols} needed")
    if t.dim() == 2 or t.shape[1] > 1:
        stride = t.stride(-2)
    else:
        stride = t.stride(0)
    return max(stride, t.shape[-1]) if n == 1 else stride


def _check_planes(planes, what: str, rows: int, positions: int) -> None:
    """KV planes (or block pools) as tensors [rows, positions, ...]: all of one
    shape, strides and dtype, on the GPU, holding ``rows`` rows of
    ``positions`` positions."""
    p0 = planes[0]
    for i, p in enumerate(planes):
        if not p.is_cuda:
            raise ValueError(f"{what} {i}: a GPU tensor is needed")
        if p.shape != p0.shape or p.stride() != p0.stride() or p.dtype != p0.dtype:
            raise ValueError(f"{what} {i}: every plane must have the shape, strides and dtype "
                             f"of the first")
    if p0.dim() < 2 or p0.shape[0] < rows or p0.shape[1] < positions:
        raise ValueError(f"{what}: shape {tuple(p0.shape)}, at least [{rows}, {positions}, ...] "
                         f"needed")
    if p0[0, 0].numel() != 1 and not p0[0, 0].is_contiguous():
        raise ValueError(f"{what}: the elements of a position must be contiguous")


def _torch_int32():
    import torch
    return torch.int32


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# the C ABI, one function each
# ---------------------------------------------------------------------------

def bs_strerror(status: int) -> str:
    return library().bs_strerror(status).decode()


def bs_create(cfg: bs_config, stream=None) -> int:
    h = ctypes.c_void_p()
    _check(library().bs_create(ctypes.byref(cfg), _stream(stream), ctypes.byref(h)), "bs_create")
    return h.value


def bs_reset(h: int) -> None:
    _check(library().bs_reset(h), "bs_reset")


def bs_step(h: int, logits, beam_idx, token_id, scores, done) -> None:
    _check(library().bs_step(h, _ptr(logits), _rows(logits, "logits"), _ptr(beam_idx),
                             _ptr(token_id), _ptr(scores), _ptr(done)), "bs_step")


def make_kv_desc(planes: Sequence, pos_offset: int = 0) -> bs_kv_desc:
    """Descriptor of planes that are torch tensors [rows, positions, ...]."""
    p0 = planes[0]
    es = p0.element_size()
    arr = (ctypes.c_void_p * len(planes))(*[p.data_ptr() for p in planes])
    d = bs_kv_desc(len(planes), ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)),
                   p0.stride(0) * es, p0.stride(1) * es, pos_offset,
                   p0[0, 0].numel() * es)
    d._keep = arr  # the pointer array must outlive the call
    return d


def bs_reorder_kv(h: int, kv: bs_kv_desc, gen_len: int) -> None:
    _check(library().bs_reorder_kv(h, ctypes.byref(kv), gen_len), "bs_reorder_kv")


def bs_reorder_kv_timed(h: int, kv: bs_kv_desc, gen_len: int, start_event: int,
                        stop_event: int) -> None:
    """bs_reorder_kv with hipEvent_t handles (ints, 0 for none) attached to
    its first and last kernel dispatch."""
    _check(library().bs_reorder_kv_timed(h, ctypes.byref(kv), gen_len, start_event or None,
                                         stop_event or None), "bs_reorder_kv_timed")


def bs_kv_paged_create(h: int, block_size: int, blocks_per_item: int) -> int:
    p = ctypes.c_void_p()
    _check(library().bs_kv_paged_create(h, block_size, blocks_per_item, ctypes.byref(p)),
           "bs_kv_paged_create")
    return p.value


def bs_kv_paged_reset(p: int) -> None:
    _check(library().bs_kv_paged_reset(p), "bs_kv_paged_reset")


def bs_kv_paged_table(p: int):
    """(device address of the table, max_blocks)."""
    t, mb = ctypes.c_void_p(), ctypes.c_int32()
    _check(library().bs_kv_paged_table(p, ctypes.byref(t), ctypes.byref(mb)), "bs_kv_paged_table")
    return t.value, mb.value


def make_kv_pool(pools: Sequence) -> bs_kv_pool:
    """Descriptor of block pools that are torch tensors [blocks, block_size, ...]."""
    p0 = pools[0]
    es = p0.element_size()
    arr = (ctypes.c_void_p * len(pools))(*[p.data_ptr() for p in pools])
    d = bs_kv_pool(len(pools), ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)),
                   p0.stride(0) * es, p0.stride(1) * es, p0[0, 0].numel() * es)
    d._keep = arr  # the pointer array must outlive the call
    return d


def bs_kv_paged_reorder(p: int, pool: bs_kv_pool, gen_len: int) -> None:
    _check(library().bs_kv_paged_reorder(p, ctypes.byref(pool), gen_len), "bs_kv_paged_reorder")


def bs_kv_paged_status(p: int, batch: int):
    """(overflow flag, free blocks per item as a list); synchronises."""
    ov = ctypes.c_int32()
    fb = (ctypes.c_int32 * batch)()
    _check(library().bs_kv_paged_status(p, ctypes.byref(ov), fb), "bs_kv_paged_status")
    return ov.value, list(fb)


def bs_kv_paged_destroy(p: int) -> None:
    library().bs_kv_paged_destroy(p)


def bs_finalize(h: int, tokens, lengths, norm_scores) -> None:
    _check(library().bs_finalize(h, _ptr(tokens), _ptr(lengths), _ptr(norm_scores)),
           "bs_finalize")


def bs_last_selection(h: int, flat_idx, cand_score) -> None:
    _check(library().bs_last_selection(h, _ptr(flat_idx), _ptr(cand_score)),
           "bs_last_selection")


def bs_get_finished(h: int, norm, raw, length, step, rank, count) -> None:
    _check(library().bs_get_finished(h, _ptr(norm), _ptr(raw), _ptr(length), _ptr(step),
                                     _ptr(rank), _ptr(count)), "bs_get_finished")


def bs_steps_taken(h: int) -> int:
    return library().bs_steps_taken(h)


def bs_state_size(h: int) -> int:
    n = ctypes.c_int64()
    _check(library().bs_state_size(h, ctypes.byref(n)), "bs_state_size")
    return n.value


def bs_state_save(h: int) -> bytes:
    """The handle's search state as a snapshot (host bytes); synchronises."""
    n = bs_state_size(h)
    buf = ctypes.create_string_buffer(n)
    _check(library().bs_state_save(h, buf, n), "bs_state_save")
    return buf.raw


def bs_state_load(h: int, snapshot: bytes) -> None:
    buf = ctypes.create_string_buffer(snapshot, len(snapshot))
    _check(library().bs_state_load(h, buf, len(snapshot)), "bs_state_load")


def bs_destroy(h: int) -> None:
    library().bs_destroy(h)


def bs_verify_create(batch: int, k: int, vocab: int, dtype: int, stream=None) -> int:
    h = ctypes.c_void_p()
    _check(library().bs_verify_create(batch, k, vocab, dtype, _stream(stream), ctypes.byref(h)),
           "bs_verify_create")
    return h.value


def _verify_stride(logits) -> int:
    """Row stride in elements of logits [B*k, S] or [B, k, S] (rows evenly spaced)."""
    return _rows(logits, "logits")


def bs_verify(h: int, logits, proposals, accept_len, argmax) -> None:
    _check(library().bs_verify(h, _ptr(logits), _verify_stride(logits), _ptr(proposals),
                               _ptr(accept_len), _ptr(argmax)), "bs_verify")


def bs_verify_ex(h: int, logits, proposals, top_k: int, min_block: int, accept_len, argmax,
                 prop_rank=None) -> None:
    _check(library().bs_verify_ex(h, _ptr(logits), _verify_stride(logits), _ptr(proposals),
                                  top_k, min_block, _ptr(accept_len), _ptr(argmax),
                                  _ptr(prop_rank) if prop_rank is not None else None),
           "bs_verify_ex")


def bs_verify_noalloc(logits, dtype: int, batch: int, k: int, vocab: int, proposals, accept_len,
                      argmax, stream=None) -> None:
    """The verify call with the library's static workspace (no handle, no
    allocation); logits [B*k, S] or [B, k, S]."""
    _check(library().bs_verify_noalloc(_stream(stream), _ptr(logits), dtype, batch, k, vocab,
                                       _verify_stride(logits), _ptr(proposals),
                                       _ptr(accept_len), _ptr(argmax)), "bs_verify_noalloc")


def bs_verify_destroy(h: int) -> None:
    library().bs_verify_destroy(h)


# ---------------------------------------------------------------------------
# convenience wrapper owning the handle and the output tensors
# ---------------------------------------------------------------------------

class BeamSearch:
    """One batched beam search on the current GPU.

    ``step(logits)`` runs expand/score/prune/finalize; ``reorder_kv(planes,
    gen_len)`` moves the KV cache rows that changed parent; ``finalize()``
    returns the best hypotheses. Outputs are torch tensors on the device.
    """

    def __init__(self, batch, beam, vocab, max_steps, eos_id=-1, pad_id=-1, dtype="f32",
                 lp="gnmt", alpha=0.6, stop="heuristic", num_return=1, tile_elems=0,
                 prune="topw", select="fused", stream=None):
        import torch
        self.B, self.W, self.V, self.T = batch, beam, vocab, max_steps
        self.dtype = dtype
        self.K = 2 * beam if prune == "top2w" else beam   # candidates ranked per item
        self.num_return = num_return
        self.cfg = bs_config(batch, beam, vocab, max_steps, eos_id, pad_id, DTYPES[dtype],
                             LPS[lp], float(alpha), STOPS[stop], num_return, tile_elems,
                             PRUNES[prune], SELECTS[select])
        self.stream = stream
        self.h = bs_create(self.cfg, stream)
        dev = torch.device("cuda", torch.cuda.current_device())
        self.beam_idx = torch.empty((batch, beam), dtype=torch.int32, device=dev)
        self.token_id = torch.empty((batch, beam), dtype=torch.int32, device=dev)
        self.scores = torch.empty((batch, beam), dtype=torch.float32, device=dev)
        self.done = torch.empty(batch, dtype=torch.uint8, device=dev)
        self.device = dev

    @classmethod
    def for_workload(cls, wl, **over):
        kw = dict(batch=wl.batch, beam=wl.beam, vocab=wl.vocab, max_steps=wl.max_steps,
                  eos_id=wl.eos_id, pad_id=wl.pad_id, dtype=wl.dtype, lp=wl.lp,
                  alpha=wl.alpha, stop=wl.stop, num_return=wl.num_return)
        kw.update(over)
        return cls(**kw)

    def close(self):
        if getattr(self, "h", None):
            bs_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self):
        bs_reset(self.h)

    def save(self) -> bytes:
        """A snapshot of the search (host bytes), to resume it with load()."""
        return bs_state_save(self.h)

    def load(self, snapshot: bytes) -> None:
        bs_state_load(self.h, snapshot)

    @property
    def steps(self) -> int:
        return bs_steps_taken(self.h)

    def step(self, logits):
        _rows(logits, "logits", self.B * self.W, self.V, LOGIT_DTYPES[self.dtype])
        bs_step(self.h, logits, self.beam_idx, self.token_id, self.scores, self.done)
        return self.beam_idx, self.token_id, self.scores, self.done

    def reorder_kv(self, planes_or_desc, gen_len: int, pos_offset: int = 0):
        d = planes_or_desc
        if not isinstance(d, bs_kv_desc):
            _check_planes(d, "KV plane", self.B * self.W, pos_offset + gen_len)
            d = make_kv_desc(d, pos_offset)
        bs_reorder_kv(self.h, d, gen_len)

    def selection(self):
        import torch
        j = torch.empty((self.B, self.K), dtype=torch.int32, device=self.device)
        c = torch.empty((self.B, self.K), dtype=torch.float32, device=self.device)
        bs_last_selection(self.h, j, c)
        return j, c

    def finished(self):
        import torch
        kw = dict(device=self.device)
        norm = torch.empty((self.B, self.W), dtype=torch.float32, **kw)
        raw = torch.empty_like(norm)
        ln = torch.empty((self.B, self.W), dtype=torch.int32, **kw)
        st, rk = torch.empty_like(ln), torch.empty_like(ln)
        cnt = torch.empty(self.B, dtype=torch.int32, **kw)
        bs_get_finished(self.h, norm, raw, ln, st, rk, cnt)
        return norm, raw, ln, st, rk, cnt

    def finalize(self):
        import torch
        R = self.num_return
        tok = torch.empty((self.B, R, self.T), dtype=torch.int32, device=self.device)
        ln = torch.empty((self.B, R), dtype=torch.int32, device=self.device)
        nm = torch.empty((self.B, R), dtype=torch.float32, device=self.device)
        bs_finalize(self.h, tok, ln, nm)
        return tok, ln, nm


class PagedKV:
    """Block tables with copy on write for a BeamSearch's KV cache.

    ``table()`` returns a copy of the device table as a torch tensor
    [B*W, max_blocks]; ``reorder(pools, t)`` follows the bs_step of step t.
    """

    def __init__(self, search: "BeamSearch", block_size: int, blocks_per_item: int = 0):
        self.search = search
        self.block_size = block_size
        mb = search.T // block_size + 1 if block_size >= 1 else 1
        self.blocks_per_item = blocks_per_item or search.W * mb
        self.h = bs_kv_paged_create(search.h, block_size, self.blocks_per_item)
        self._addr, self.max_blocks = bs_kv_paged_table(self.h)

    def table(self):
        """A copy of the device table as a torch int32 tensor [B*W, max_blocks],
        taken after the handle's stream has reached it."""
        import torch
        t = torch.empty((self.search.B * self.search.W, self.max_blocks), dtype=torch.int32,
                        device=self.search.device)
        torch.cuda.synchronize(self.search.device)
        _hip_copy_d2d(t.data_ptr(), self._addr, t.numel() * 4)
        return t

    def reset(self):
        bs_kv_paged_reset(self.h)

    def reorder(self, pools_or_desc, gen_len: int):
        d = pools_or_desc
        if not isinstance(d, bs_kv_pool):
            _check_planes(d, "block pool", self.search.B * self.blocks_per_item, self.block_size)
            d = make_kv_pool(d)
        bs_kv_paged_reorder(self.h, d, gen_len)

    def status(self):
        return bs_kv_paged_status(self.h, self.search.B)

    def close(self):
        if getattr(self, "h", None):
            bs_kv_paged_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _hip_copy_d2d(dst: int, src: int, nbytes: int) -> None:
    """Synchronous device-to-device copy through the HIP runtime torch loaded."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    rc = hip.hipMemcpy(dst, src, nbytes, 3)  # hipMemcpyDeviceToDevice
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed ({rc})")


class Verifier:
    """Blockwise-parallel verify for logits [B, k, V] on the current GPU."""

    def __init__(self, batch, k, vocab, dtype="f32", stream=None):
        import torch
        self.B, self.k, self.V = batch, k, vocab
        self.dtype = dtype
        self.h = bs_verify_create(batch, k, vocab, DTYPES[dtype], stream)
        dev = torch.device("cuda", torch.cuda.current_device())
        self.accept_len = torch.empty(batch, dtype=torch.int32, device=dev)
        self.argmax = torch.empty((batch, k), dtype=torch.int32, device=dev)

    def close(self):
        if getattr(self, "h", None):
            bs_verify_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __call__(self, logits, proposals, top_k=1, min_block=0, rank=False):
        """Exact verify by default; top_k > 1 or min_block > 1 gives the
        approximate criteria. With rank=True also returns each proposal's rank."""
        _rows(logits, "logits", self.B * self.k, self.V, LOGIT_DTYPES[self.dtype])
        if not proposals.is_cuda or proposals.dtype != _torch_int32() or \
                not proposals.is_contiguous() or proposals.numel() < self.B * self.k:
            raise ValueError(f"proposals: a contiguous GPU int32 tensor of {self.B * self.k} "
                             f"elements is needed")
        if top_k == 1 and min_block == 0 and not rank:
            bs_verify(self.h, logits, proposals, self.accept_len, self.argmax)
            return self.accept_len, self.argmax
        import torch
        rk = None
        if rank:
            rk = torch.empty((self.B, self.k), dtype=torch.int32, device=self.argmax.device)
        bs_verify_ex(self.h, logits, proposals, top_k, min_block, self.accept_len, self.argmax,
                     rk)
        return (self.accept_len, self.argmax, rk) if rank else (self.accept_len, self.argmax)
