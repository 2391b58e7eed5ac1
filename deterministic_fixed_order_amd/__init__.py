"""Deterministic fixed-order fold on AMD Instinct MI355X -- Python binding.

A thin ctypes layer over ``libdetfold.so`` (C ABI in ``include/detfold.h``).
It only marshals arguments: it checks tensor dtype, device, shape and
contiguity, passes raw device pointers and the caller's current HIP stream,
and raises on a nonzero return code.  Every step of the fold runs in the HIP
kernels; there is no CPU fallback, and importing a function whose library is
missing raises.

PyTorch is used for device memory and streams only.

    fold_ranks(out, stacked)                 out = s_0 + s_1 + ... + s_{W-1}, ascending
    fold_ranks_scaled(out, stacked, inv_w)   the same, then * inv_w
    fold_into(dst, stage)                    dst = dst + stage (in place)
    fold_slots(out, [s_0, ..., s_{W-1}])     the fold over separate buffers (W <= 16)
    fold_ranks_batch(outs, stackeds)         many stacked folds of one width in one launch
    loopback_round(arenas, stage=None, ...)  one reduction round over W arenas (staged, direct, fused)
    PairLink(...).all_reduce(x0, x1)         two-stream (two-rank) all-reduce on one device
    PairLink(...).broadcast / all_gather     pure movement between the two ranks
    OneShotLink(...).all_reduce(x0, x1)      the one-kernel arm with an in-kernel barrier

``stacked`` is a ``[W, len]`` float32 CUDA/HIP tensor (row r = slot r); a view
with a storage offset is fine as long as it is contiguous.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdetfold.so")

OK, EINVAL, EOVERLAP, ELAUNCH, EDEVICE, ESIZE, ECAPTURE = 0, 1, 2, 3, 4, 5, 6
PATH_AUTO, PATH_VECTOR, PATH_SCALAR, PATH_ROWS = 0, 1, 2, 3
POLICY_DEFAULT, POLICY_STREAM, POLICY_CACHED = 0, 1, 2
ABI_VERSION = 12
STATIC_STAGE_FLOATS = 1 << 22
ONE_SHOT_BLOCKS = 64
ONE_SHOT_FLAG_WORDS = 2 * 2 * ONE_SHOT_BLOCKS
BARRIER_ENTRY_EXPIRED, BARRIER_EXIT_EXPIRED = 40043, 40044
ROUND_REVERSE_DELIVERY, ROUND_DIRECT, ROUND_FUSED = 1, 2, 4

EXPORTS = (
    "fold_ranks", "fold_into", "fold_ranks_scaled", "detfold_strerror", "detfold_abi_version",
    "detfold_shard_plan", "detfold_plan_fold_ranks", "detfold_plan_fold_into",
    "detfold_fold_ranks_ex", "fold_slots", "fold_slots_scaled", "detfold_loopback_round",
    "detfold_pair_link_init", "detfold_pair_all_reduce", "detfold_pair_broadcast",
    "detfold_pair_all_gather", "detfold_one_shot_init", "detfold_one_shot_all_reduce",
    "detfold_one_shot_rank", "detfold_fold_ranks_timed", "detfold_loopback_round_static",
    "fold_ranks_batch", "fold_ranks_batch_scaled", "detfold_plan_fold_ranks_batch",
)
MAX_JOBS = 32


class DetfoldError(RuntimeError):
    def __init__(self, rc: int, what: str):
        self.rc = rc
        super().__init__("%s: detfold rc=%d (%s)" % (what, rc, strerror(rc)))


class Launch(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("block", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("unroll", ctypes.c_int32), ("policy", ctypes.c_int32),
                ("group", ctypes.c_int32)]


class FoldJob(ctypes.Structure):
    _fields_ = [("out", ctypes.c_void_p), ("stacked", ctypes.c_void_p), ("len", ctypes.c_int64),
                ("pitch", ctypes.c_int64)]


class PairLinkC(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p * 2), ("stage", ctypes.c_void_p * 2),
                ("capacity", ctypes.c_int64), ("pushed", ctypes.c_void_p * 2),
                ("folded", ctypes.c_void_p * 2)]


class OneShotLinkC(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("stage", ctypes.c_void_p * 2),
                ("capacity", ctypes.c_int64), ("flags", ctypes.c_void_p), ("words", ctypes.c_void_p),
                ("spin_limit", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("block", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("unroll", ctypes.c_int32), ("head", ctypes.c_int32), ("tail", ctypes.c_int32),
                ("policy", ctypes.c_int32), ("body", ctypes.c_int64), ("tile", ctypes.c_int64),
                ("group", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load ``libdetfold.so``; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            "libdetfold.so is not built at %s; run `python -c 'import __graft_entry__ as g; "
            "g.build()'` from the repository root" % path)
    lib = ctypes.CDLL(path)
    vp, f32p, i32, i64 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.fold_ranks.argtypes = [f32p, f32p, i32, i64, vp]
    lib.fold_into.argtypes = [f32p, f32p, i64, vp]
    lib.fold_ranks_scaled.argtypes = [f32p, f32p, i32, i64, ctypes.c_float, vp]
    lib.detfold_fold_ranks_ex.argtypes = [f32p, f32p, i32, i64, i32, ctypes.c_float,
                                          ctypes.POINTER(Launch), vp]
    lib.detfold_fold_ranks_timed.argtypes = [f32p, f32p, i32, i64, i32, ctypes.c_float,
                                             ctypes.POINTER(Launch), vp, vp, vp]
    lib.detfold_strerror.argtypes = [ctypes.c_int]
    lib.detfold_strerror.restype = ctypes.c_char_p
    lib.detfold_abi_version.argtypes = []
    lib.detfold_shard_plan.argtypes = [i64, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    # uintptr_t addresses: size_t has the same width on the supported hosts
    lib.detfold_plan_fold_ranks.argtypes = [ctypes.c_size_t, ctypes.c_size_t, i32, i64, i32,
                                            ctypes.POINTER(Launch), ctypes.POINTER(Plan)]
    lib.detfold_plan_fold_into.argtypes = [ctypes.c_size_t, ctypes.c_size_t, i64, i32,
                                           ctypes.POINTER(Plan)]
    pp = ctypes.POINTER(ctypes.c_void_p)
    lib.fold_slots.argtypes = [f32p, pp, i32, i64, vp]
    lib.fold_slots_scaled.argtypes = [f32p, pp, i32, i64, ctypes.c_float, vp]
    lib.detfold_loopback_round.argtypes = [pp, i32, i64, f32p, i64, i32, vp]
    lib.detfold_loopback_round_static.argtypes = [pp, i32, i64, i32, vp]
    jp = ctypes.POINTER(FoldJob)
    lib.fold_ranks_batch.argtypes = [jp, i32, i32, vp]
    lib.fold_ranks_batch_scaled.argtypes = [jp, i32, i32, ctypes.c_float, vp]
    lib.detfold_plan_fold_ranks_batch.argtypes = [jp, i32, i32, i32, ctypes.POINTER(Plan)]
    lib.detfold_pair_link_init.argtypes = [ctypes.POINTER(PairLinkC)]
    lib.detfold_pair_all_reduce.argtypes = [ctypes.POINTER(PairLinkC), f32p, f32p, i64]
    lib.detfold_pair_broadcast.argtypes = [ctypes.POINTER(PairLinkC), i32, f32p, f32p, i64]
    lib.detfold_pair_all_gather.argtypes = [ctypes.POINTER(PairLinkC), f32p, f32p, f32p, f32p, i64]
    lib.detfold_one_shot_init.argtypes = [ctypes.POINTER(OneShotLinkC)]
    lib.detfold_one_shot_all_reduce.argtypes = [ctypes.POINTER(OneShotLinkC), f32p, f32p, i64]
    lib.detfold_one_shot_rank.argtypes = [ctypes.POINTER(OneShotLinkC), i32, f32p, i64, vp]
    for name in EXPORTS:
        if name != "detfold_strerror":
            getattr(lib, name).restype = ctypes.c_int
    if lib.detfold_abi_version() != ABI_VERSION:
        raise RuntimeError("libdetfold ABI mismatch")
    _lib = lib
    return lib


def strerror(rc: int) -> str:
    return load().detfold_strerror(rc).decode()


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise DetfoldError(rc, what)


_raw_current_stream = None


def _stream_handle(t, stream) -> int:
    """The hipStream_t to enqueue on: `stream` if given, else the caller's
    current stream on t's device.  torch's raw accessor returns the handle
    directly (0.1 us against 2 us for building a Stream object); the public
    call is the fallback where it is missing."""
    global _raw_current_stream
    if stream is not None:
        return int(stream.cuda_stream)
    if _raw_current_stream is None:
        import torch
        _raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _raw_current_stream:
        return int(_raw_current_stream(t.device.index))
    import torch
    return int(torch.cuda.current_stream(t.device).cuda_stream)


def _f32_device(t, name: str) -> None:
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32, got %s" % (name, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stacked_shape(out, stacked):
    _f32_device(out, "out")
    _f32_device(stacked, "stacked")
    if stacked.dim() != 2:
        raise ValueError("stacked must be [W, len], got shape %s" % (tuple(stacked.shape),))
    W, n = stacked.shape
    if out.numel() != n:
        raise ValueError("out has %d elements, stacked rows have %d" % (out.numel(), n))
    if out.device != stacked.device:
        raise ValueError("out and stacked are on different devices")
    return int(W), int(n)


def fold_ranks(out, stacked, stream=None) -> None:
    """``out[i] = ((stacked[0,i] + stacked[1,i]) + ...) + stacked[W-1,i]``."""
    W, n = _stacked_shape(out, stacked)
    _check(load().fold_ranks(out.data_ptr(), stacked.data_ptr(), W, n,
                             _stream_handle(out, stream)), "fold_ranks")


def fold_ranks_scaled(out, stacked, inv_w: float, stream=None) -> None:
    """``fold_ranks`` followed by one binary32 multiply of each sum by ``inv_w``."""
    W, n = _stacked_shape(out, stacked)
    _check(load().fold_ranks_scaled(out.data_ptr(), stacked.data_ptr(), W, n, float(inv_w),
                                    _stream_handle(out, stream)), "fold_ranks_scaled")


def fold_into(dst, stage, stream=None) -> None:
    """``dst[i] = dst[i] + stage[i]`` in place."""
    _f32_device(dst, "dst")
    _f32_device(stage, "stage")
    if dst.numel() != stage.numel():
        raise ValueError("dst has %d elements, stage %d" % (dst.numel(), stage.numel()))
    if dst.device != stage.device:
        raise ValueError("dst and stage are on different devices")
    _check(load().fold_into(dst.data_ptr(), stage.data_ptr(), dst.numel(),
                            _stream_handle(dst, stream)), "fold_into")


def _jobs(outs, stackeds):
    if len(outs) != len(stackeds):
        raise ValueError("%d outputs for %d arenas" % (len(outs), len(stackeds)))
    if len(outs) > MAX_JOBS:
        raise ValueError("at most %d jobs per call, got %d" % (MAX_JOBS, len(outs)))
    W = None
    jobs = (FoldJob * max(len(outs), 1))()
    for j, (out, stacked) in enumerate(zip(outs, stackeds)):
        w, n, pitch = _pitched_shape(out, stacked)
        if W is not None and w != W:
            raise ValueError("job %d has W=%d, job 0 has W=%d" % (j, w, W))
        W = w
        jobs[j].out, jobs[j].stacked, jobs[j].len, jobs[j].pitch = out.data_ptr(), stacked.data_ptr(), n, pitch
    return jobs, len(outs), (W or 1)


def _pitched_shape(out, stacked):
    """W, len and slot pitch of a [W, len] view whose rows may be padded apart
    (row stride >= len, elements contiguous within a row)."""
    import torch
    _f32_device(out, "out")
    if not isinstance(stacked, torch.Tensor) or stacked.dtype != torch.float32:
        raise TypeError("stacked must be a float32 torch.Tensor")
    if stacked.device.type != "cuda" or stacked.device != out.device:
        raise ValueError("stacked must be a device tensor on out's device")
    if stacked.dim() != 2:
        raise ValueError("stacked must be [W, len], got shape %s" % (tuple(stacked.shape),))
    W, n = (int(x) for x in stacked.shape)
    if out.numel() != n:
        raise ValueError("out has %d elements, stacked rows have %d" % (out.numel(), n))
    if n > 1 and stacked.stride(1) != 1:
        raise ValueError("stacked rows must be contiguous")
    pitch = int(stacked.stride(0)) if W > 1 else n
    if W > 1 and pitch < n:
        raise ValueError("stacked rows overlap (row stride %d < len %d)" % (pitch, n))
    return W, n, pitch


def fold_ranks_batch(outs, stackeds, inv_w: Optional[float] = None, stream=None) -> None:
    """``fold_ranks(outs[j], stackeds[j])`` for every j (same W), in one launch
    where 2 <= W <= 16; with ``inv_w``, ``fold_ranks_scaled`` instead.  Each
    ``stackeds[j]`` is a [W, len] view whose rows may be padded apart (for
    instance ``buf.view(W, pitch)[:, :len]``)."""
    jobs, count, W = _jobs(outs, stackeds)
    if count == 0:
        return
    h = _stream_handle(outs[0], stream)
    if inv_w is None:
        _check(load().fold_ranks_batch(jobs, count, W, h), "fold_ranks_batch")
    else:
        _check(load().fold_ranks_batch_scaled(jobs, count, W, float(inv_w), h), "fold_ranks_batch_scaled")


def fold_ranks_ex(out, stacked, *, scaled: bool = False, inv_w: float = 1.0, path: int = 0,
                  block: int = 0, grid: int = 0, unroll: int = 0, policy: int = 0, group: int = 0,
                  stream=None) -> None:
    """``fold_ranks`` / ``fold_ranks_scaled`` with an explicit launch override
    (tests and tuning sweeps only)."""
    W, n = _stacked_shape(out, stacked)
    cfg = Launch(path, block, grid, unroll, policy, group)
    _check(load().detfold_fold_ranks_ex(out.data_ptr(), stacked.data_ptr(), W, n, int(scaled),
                                        float(inv_w), ctypes.byref(cfg),
                                        _stream_handle(out, stream)), "detfold_fold_ranks_ex")


def fold_ranks_timed(out, stacked, start, stop, *, scaled: bool = False, inv_w: float = 1.0,
                     launch: Optional[dict] = None, stream=None) -> None:
    """``fold_ranks`` / ``fold_ranks_scaled`` whose kernel dispatch records the
    timing-enabled ``torch.cuda.Event`` objects ``start`` and ``stop`` itself
    (measurement only): ``start.elapsed_time(stop)`` is the kernel's own
    duration.  Both events must have been recorded once before, so that their
    device events exist."""
    W, n = _stacked_shape(out, stacked)
    handles = []
    for e, nm in ((start, "start"), (stop, "stop")):
        h = int(e.cuda_event) if e is not None else 0
        if e is not None and not h:
            raise ValueError("%s has no device event yet; record it once first" % nm)
        handles.append(h or None)
    cfg = ctypes.byref(Launch(**launch)) if launch else None
    _check(load().detfold_fold_ranks_timed(out.data_ptr(), stacked.data_ptr(), W, n, int(scaled),
                                           float(inv_w), cfg, _stream_handle(out, stream),
                                           handles[0], handles[1]), "detfold_fold_ranks_timed")


def _ptr_array(tensors):
    return (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])


def _same_len_slots(out, slots):
    _f32_device(out, "out")
    if not slots:
        raise ValueError("need at least one slot")
    for i, t in enumerate(slots):
        _f32_device(t, "slots[%d]" % i)
        if t.numel() != out.numel():
            raise ValueError("slot %d has %d elements, out %d" % (i, t.numel(), out.numel()))
        if t.device != out.device:
            raise ValueError("slot %d is on another device" % i)


def fold_slots(out, slots, stream=None) -> None:
    """``out = ((slots[0] + slots[1]) + ...) + slots[W-1]`` over separate tensors
    (W <= 16); ``out`` may be one of the slots (in place)."""
    _same_len_slots(out, slots)
    _check(load().fold_slots(out.data_ptr(), _ptr_array(slots), len(slots), out.numel(),
                             _stream_handle(out, stream)), "fold_slots")


def fold_slots_scaled(out, slots, inv_w: float, stream=None) -> None:
    """``fold_slots`` followed by one binary32 multiply by ``inv_w``."""
    _same_len_slots(out, slots)
    _check(load().fold_slots_scaled(out.data_ptr(), _ptr_array(slots), len(slots), out.numel(),
                                    float(inv_w), _stream_handle(out, stream)), "fold_slots_scaled")


def round_stage_elems(n: int, world: int) -> int:
    """Floats of staging a staged ``loopback_round`` needs: W * ceil(n / W)."""
    return world * (-(-n // world)) if world > 0 else 0


def loopback_round(arenas, stage=None, *, reverse_delivery: bool = False, direct: bool = False,
                   fused: bool = False, stream=None) -> None:
    """One fixed-order reduction round across the W arenas (one device).

    Afterwards every arena holds the ascending-rank fold of all the arenas'
    previous contents.  Staged (default) gathers each owner's shard copies into
    ``stage`` (at least ``round_stage_elems(n, W)`` floats) before folding;
    ``direct`` folds each owner's shard straight from the arenas, then
    distributes it; ``fused`` does the whole round in one kernel that folds
    every tile from the arenas and writes it back into all of them."""
    if not arenas:
        raise ValueError("need at least one arena")
    n = arenas[0].numel()
    for i, a in enumerate(arenas):
        _f32_device(a, "arenas[%d]" % i)
        if a.numel() != n:
            raise ValueError("arena %d has %d elements, arena 0 has %d" % (i, a.numel(), n))
    flags = ((ROUND_REVERSE_DELIVERY if reverse_delivery else 0) | (ROUND_DIRECT if direct else 0)
             | (ROUND_FUSED if fused else 0))
    stage_ptr, stage_elems = None, 0
    if stage is not None:
        _f32_device(stage, "stage")
        stage_ptr, stage_elems = stage.data_ptr(), stage.numel()
    _check(load().detfold_loopback_round(_ptr_array(arenas), len(arenas), n, stage_ptr, stage_elems,
                                         flags, _stream_handle(arenas[0], stream)),
           "loopback_round")


def loopback_round_static(arenas, *, reverse_delivery: bool = False, stream=None) -> None:
    """The staged ``loopback_round`` with the library's own static stage
    (``STATIC_STAGE_FLOATS`` floats per device): nothing is allocated.  W *
    ceil(n / W) must fit the stage (else ``ESIZE``); calls that overlap in time
    on one device race on the stage."""
    if not arenas:
        raise ValueError("need at least one arena")
    n = arenas[0].numel()
    for i, a in enumerate(arenas):
        _f32_device(a, "arenas[%d]" % i)
        if a.numel() != n:
            raise ValueError("arena %d has %d elements, arena 0 has %d" % (i, a.numel(), n))
    _check(load().detfold_loopback_round_static(_ptr_array(arenas), len(arenas), n,
                                                ROUND_REVERSE_DELIVERY if reverse_delivery else 0,
                                                _stream_handle(arenas[0], stream)),
           "loopback_round_static")


class PairLink:
    """Two ranks on one device, each a stream, joined by staging buffers and
    events (the library's ``detfold_pair_link``).  ``all_reduce(x0, x1)`` leaves
    ``x0 + x1`` in both, folded on each rank's own stream.

    Stream order: every call first makes both rank streams wait for the
    caller's current stream (so work already queued there on the tensors,
    such as the writes that produced them, comes first), and before it
    returns makes the current stream wait for the events that mark the end of
    the call's last work on each rank stream -- the ones the library's
    dispatches record (``folded`` after an all-reduce, ``pushed`` after the
    movement calls) -- so later work there, including the allocator's reuse
    of a freed tensor, comes after.  One event recorded on the current
    stream serves both rank streams, and the join records none: each
    recorded event costs the host several microseconds.  Between the two the
    ranks run on their own streams.

    The link cannot be captured into a HIP graph (the library returns
    ``ECAPTURE``); every call raises before touching the device while the
    current stream is capturing."""

    def __init__(self, capacity: int, device=None, streams=None):
        import torch
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.streams = list(streams) if streams is not None else [torch.cuda.Stream(device=dev) for _ in range(2)]
        self.stage = [torch.empty(max(capacity, 1), dtype=torch.float32, device=dev) for _ in range(2)]
        # timing disabled: the events only order the two streams
        self.pushed = [torch.cuda.Event(enable_timing=False) for _ in range(2)]
        self.folded = [torch.cuda.Event(enable_timing=False) for _ in range(2)]
        for e in self.pushed + self.folded:
            e.record(self.streams[0])  # materialise the underlying event
        # marks the caller's stream for both rank streams at each call's start
        self._entry = torch.cuda.Event(enable_timing=False)
        self._ranks = [self.streams[0]] if self.streams[1] == self.streams[0] else list(self.streams)
        torch.cuda.synchronize(dev)
        self.capacity = capacity
        self._c = PairLinkC()
        for r in range(2):
            self._c.stream[r] = self.streams[r].cuda_stream
            self._c.stage[r] = self.stage[r].data_ptr()
            self._c.pushed[r] = self.pushed[r].cuda_event  # the raw hipEvent_t
            self._c.folded[r] = self.folded[r].cuda_event
        self._c.capacity = capacity
        _check(load().detfold_pair_link_init(ctypes.byref(self._c)), "pair_link_init")

    def _fork(self):
        import torch
        if torch.cuda.is_current_stream_capturing():
            raise DetfoldError(ECAPTURE, "PairLink")
        cur = torch.cuda.current_stream(self.device)
        self._entry.record(cur)
        for s in self._ranks:
            s.wait_event(self._entry)
        return cur

    @staticmethod
    def _join(cur, marks) -> None:
        """The current stream waits for the events that end the call's work on
        the rank streams."""
        for e in marks:
            cur.wait_event(e)

    def all_reduce(self, x0, x1) -> None:
        _f32_device(x0, "x0")
        _f32_device(x1, "x1")
        if x0.numel() != x1.numel():
            raise ValueError("x0 has %d elements, x1 %d" % (x0.numel(), x1.numel()))
        cur = self._fork()
        _check(load().detfold_pair_all_reduce(ctypes.byref(self._c), x0.data_ptr(), x1.data_ptr(),
                                              x0.numel()), "pair_all_reduce")
        self._join(cur, self.folded)  # each rank's fold is its stream's last work

    def broadcast(self, root: int, src, dst) -> None:
        """``dst`` (rank ``1 - root``) becomes a byte copy of ``src`` (rank ``root``)."""
        _f32_device(src, "src")
        _f32_device(dst, "dst")
        if src.numel() != dst.numel():
            raise ValueError("src has %d elements, dst %d" % (src.numel(), dst.numel()))
        cur = self._fork()
        _check(load().detfold_pair_broadcast(ctypes.byref(self._c), int(root), src.data_ptr(),
                                             dst.data_ptr(), src.numel()), "pair_broadcast")
        self._join(cur, [self.pushed[int(root)]])  # the copy; the other stream only waits for it

    def all_gather(self, x0, x1, f0, f1) -> None:
        """``f0`` and ``f1`` (2 * span floats) both become ``[x0 | x1]``."""
        for t, nm in ((x0, "x0"), (x1, "x1"), (f0, "f0"), (f1, "f1")):
            _f32_device(t, nm)
        span = x0.numel()
        if x1.numel() != span or f0.numel() != 2 * span or f1.numel() != 2 * span:
            raise ValueError("all_gather needs x0, x1 of one span and f0, f1 of twice it")
        cur = self._fork()
        _check(load().detfold_pair_all_gather(ctypes.byref(self._c), x0.data_ptr(), x1.data_ptr(),
                                              f0.data_ptr(), f1.data_ptr(), span), "pair_all_gather")
        self._join(cur, self.pushed)  # each rank's copy; after it a stream only waits


class OneShotLink:
    """The one-kernel two-rank all-reduce (the library's ``detfold_one_shot_link``):
    staging buffers, device barrier counters and two barrier words.

    ``all_reduce(x0, x1)`` runs both ranks in one launch; ``rank(r, x)`` runs
    rank r's kernel alone (both ranks must then be launched, with the same n).
    ``barrier_words()`` reads the two words: 0, or ``BARRIER_ENTRY_EXPIRED`` /
    ``BARRIER_EXIT_EXPIRED`` when a wait ran out of polls."""

    def __init__(self, capacity: int, device=None, stream=None, spin_limit: int = 0,
                 buffers=None, init: bool = True):
        """``buffers``: an existing link's ``(stage, flags, words)`` -- for
        instance tensors shared from another process -- used in place of new
        ones; ``init=False`` then leaves their counters as they are."""
        import torch
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.stream = stream if stream is not None else torch.cuda.current_stream(dev)
        if buffers is None:
            self.stage = [torch.empty(max(capacity, 1), dtype=torch.float32, device=dev) for _ in range(2)]
            self.flags = torch.empty(ONE_SHOT_FLAG_WORDS, dtype=torch.int32, device=dev)
            self.words = torch.empty(2, dtype=torch.int32, device=dev)
        else:
            stage, self.flags, self.words = buffers
            self.stage = list(stage)
            for t in self.stage:
                _f32_device(t, "stage")
                if t.numel() < capacity:
                    raise ValueError("stage holds %d floats, capacity is %d" % (t.numel(), capacity))
            if self.flags.dtype != torch.int32 or self.flags.numel() < ONE_SHOT_FLAG_WORDS:
                raise ValueError("flags must be int32 with %d words" % ONE_SHOT_FLAG_WORDS)
            if self.words.dtype != torch.int32 or self.words.numel() < 2:
                raise ValueError("words must be int32 with 2 words")
        self.capacity = capacity
        self._c = OneShotLinkC()
        self._c.stream = self.stream.cuda_stream
        for r in range(2):
            self._c.stage[r] = self.stage[r].data_ptr()
        self._c.capacity = capacity
        self._c.flags = self.flags.data_ptr()
        self._c.words = self.words.data_ptr()
        self._c.spin_limit = spin_limit
        if init:
            self.init()

    def init(self) -> None:
        """Zero the counters and words (synchronizes the link's stream)."""
        _check(load().detfold_one_shot_init(ctypes.byref(self._c)), "one_shot_init")

    def all_reduce(self, x0, x1) -> None:
        """Both ranks in one launch on the link's stream, ordered after the
        caller's current stream and before its later work (as PairLink)."""
        import torch
        _f32_device(x0, "x0")
        _f32_device(x1, "x1")
        if x0.numel() != x1.numel():
            raise ValueError("x0 has %d elements, x1 %d" % (x0.numel(), x1.numel()))
        cur = torch.cuda.current_stream(self.device)
        other = cur.cuda_stream != self.stream.cuda_stream
        if other:
            self.stream.wait_stream(cur)
        _check(load().detfold_one_shot_all_reduce(ctypes.byref(self._c), x0.data_ptr(),
                                                  x1.data_ptr(), x0.numel()), "one_shot_all_reduce")
        if other:
            cur.wait_stream(self.stream)

    def rank(self, r: int, x, stream=None) -> None:
        """Rank r's kernel alone, on ``stream`` (default: the caller's current
        stream); the caller orders it against other streams."""
        _f32_device(x, "x")
        _check(load().detfold_one_shot_rank(ctypes.byref(self._c), int(r), x.data_ptr(), x.numel(),
                                            _stream_handle(x, stream)), "one_shot_rank")

    def barrier_words(self) -> list:
        import torch
        torch.cuda.synchronize(self.device)
        return [int(v) for v in self.words.cpu().tolist()]


def shard_plan(n: int, world: int) -> list[tuple[int, int]]:
    """Contiguous owner shards ``[(start, len), ...]`` of ``[0, n)``."""
    if world < 1:
        raise DetfoldError(EINVAL, "shard_plan")
    start = (ctypes.c_int64 * world)()
    length = (ctypes.c_int64 * world)()
    _check(load().detfold_shard_plan(n, world, start, length), "shard_plan")
    return [(start[p], length[p]) for p in range(world)]


def plan_fold_ranks(out_addr: int, stacked_addr: int, W: int, n: int, cu_count: int,
                    launch: Optional[dict] = None) -> dict:
    """The plan ``fold_ranks`` would use (host only; addresses are integers)."""
    p = Plan()
    cfg = ctypes.byref(Launch(**launch)) if launch else None
    _check(load().detfold_plan_fold_ranks(out_addr, stacked_addr, W, n, cu_count, cfg,
                                          ctypes.byref(p)), "plan_fold_ranks")
    return p.as_dict()


def plan_fold_ranks_batch(jobs: list, W: int, cu_count: int) -> dict:
    """The plan of ``fold_ranks_batch``'s one launch (host only): ``jobs`` is a
    list of ``(out_addr, stacked_addr, len)`` or ``(out_addr, stacked_addr,
    len, pitch)``."""
    arr = (FoldJob * max(len(jobs), 1))()
    for j, job in enumerate(jobs):
        o, st, n = job[:3]
        arr[j].out, arr[j].stacked, arr[j].len = o, st, n
        arr[j].pitch = job[3] if len(job) > 3 else 0
    p = Plan()
    _check(load().detfold_plan_fold_ranks_batch(arr, len(jobs), W, cu_count, ctypes.byref(p)),
           "plan_fold_ranks_batch")
    return p.as_dict()


def plan_fold_into(dst_addr: int, stage_addr: int, n: int, cu_count: int) -> dict:
    """The plan ``fold_into`` would use (host only)."""
    p = Plan()
    _check(load().detfold_plan_fold_into(dst_addr, stage_addr, n, cu_count, ctypes.byref(p)),
           "plan_fold_into")
    return p.as_dict()
