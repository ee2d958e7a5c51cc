"""Python binding of libspecverify (ctypes).

Argument marshalling only: every step of verification, the budget and the
statistics runs in the HIP kernels of libspecverify.so.  torch supplies device
memory and the current stream.  There is no fallback: if the library is not
built, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecverify.so")

SV_OK = 0
SV_ERR_INVALID_ARGUMENT = 1
SV_ERR_UNSUPPORTED = 2
SV_ERR_WORKSPACE_TOO_SMALL = 3
SV_ERR_DEVICE = 4
SV_ERR_SCRATCH_TOO_SMALL = 5
SV_NOALLOC_SCRATCH_BYTES = 32 << 20

SV_DTYPE_BF16 = 0
SV_DTYPE_FP32 = 1
SV_MAX_DEPTH = 64
SV_MAX_BUDGET_POSITIONS = 4096
SV_FLAG_FORCE_FP64_DRAW = 1
SV_FLAG_STREAMING_ROW_PASS = 2
SV_FLAG_EXACT_FP64_MASSES = 4
SV_FLAG_TEAM_WAIT_GIVE_UP = 8
SV_NUM_STAGE_EVENTS = 5

BIT_BAD_DEPTH = 1
BIT_BAD_TOKEN = 2
BIT_BAD_ROW = 4
BIT_RESIDUAL_ZERO = 8
BIT_BAD_TEMPERATURE = 16
BIT_FP64_DRAW = 32
BIT_SYNC_TIMEOUT = 64

EXPORTS = ["sv_status_string", "sv_version", "sv_k_rho", "sv_allocate_budget",
           "sv_verify_workspace_bytes", "sv_verify_batch", "sv_accept_stats",
           "sv_draft_confidence_workspace_bytes", "sv_draft_confidence", "sv_select_budget_ratio",
           "sv_sample_rows", "sv_verify_batch_sharded", "sv_verify_batch_noalloc",
           "sv_stream_read", "sv_allocate_fixed_depth", "sv_accept_stats_accumulate"]
MAX_SHARDS = 16
MAX_RATIOS = 8
DCUT_RATIOS = (0.25, 0.5, 0.75, 1.0)


class SvDiag(ctypes.Structure):
    _fields_ = [("accept_margin", ctypes.c_float), ("draw_margin", ctypes.c_float),
                ("bits", ctypes.c_uint32), ("reserved", ctypes.c_int32)]


class SvVerifyArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int), ("B", ctypes.c_int32), ("D_max", ctypes.c_int32),
        ("reserved0", ctypes.c_int32), ("V", ctypes.c_int64), ("row_stride", ctypes.c_int64),
        ("target_logits", ctypes.c_void_p), ("target_row0", ctypes.c_void_p),
        ("draft_logits", ctypes.c_void_p), ("draft_row0", ctypes.c_void_p),
        ("draft_tokens", ctypes.c_void_p), ("depth", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p), ("request_id", ctypes.c_void_p),
        ("seed", ctypes.c_uint64), ("step", ctypes.c_uint32), ("flags", ctypes.c_uint32),
        ("accepted_len", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p),
        ("num_out", ctypes.c_void_p), ("alpha", ctypes.c_void_p), ("diag", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stage_events", ctypes.c_void_p), ("stats_expected_len", ctypes.c_void_p),
        ("stats_per_depth", ctypes.c_void_p), ("stats_summary", ctypes.c_void_p),
    ]


class SpecVerifyError(RuntimeError):
    pass


_lib = None


def load() -> ctypes.CDLL:
    """Load libspecverify.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise SpecVerifyError(
            f"{LIB_PATH} is missing: build it with `python -m "
            "lossless_draft_verification_softmax_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    L.sv_status_string.argtypes = [ctypes.c_int]
    L.sv_status_string.restype = ctypes.c_char_p
    L.sv_version.argtypes = []
    L.sv_version.restype = ctypes.c_char_p
    L.sv_k_rho.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_double]
    L.sv_k_rho.restype = ctypes.c_int64
    L.sv_verify_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]
    L.sv_verify_workspace_bytes.restype = ctypes.c_size_t
    L.sv_verify_batch.argtypes = [ctypes.POINTER(SvVerifyArgs), vp]
    L.sv_verify_batch.restype = ctypes.c_int
    L.sv_verify_batch_noalloc.argtypes = [ctypes.POINTER(SvVerifyArgs), vp]
    L.sv_verify_batch_noalloc.restype = ctypes.c_int
    L.sv_allocate_budget.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_int64, vp,
                                     vp, vp, vp, vp]
    L.sv_allocate_budget.restype = ctypes.c_int
    L.sv_allocate_fixed_depth.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, vp,
                                          vp, vp, vp, vp]
    L.sv_allocate_fixed_depth.restype = ctypes.c_int
    L.sv_accept_stats_accumulate.argtypes = [vp, vp, vp, ctypes.c_int32, ctypes.c_int32, vp, vp,
                                             vp]
    L.sv_accept_stats_accumulate.restype = ctypes.c_int
    L.sv_accept_stats.argtypes = [vp, vp, vp, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp]
    L.sv_accept_stats.restype = ctypes.c_int
    L.sv_draft_confidence_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                                      ctypes.c_int64]
    L.sv_draft_confidence_workspace_bytes.restype = ctypes.c_size_t
    L.sv_draft_confidence.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                      vp]
    L.sv_draft_confidence.restype = ctypes.c_int
    L.sv_select_budget_ratio.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_double), ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_int32),
                                         ctypes.POINTER(ctypes.c_float), vp, vp, vp, vp, vp, vp,
                                         vp, vp]
    L.sv_select_budget_ratio.restype = ctypes.c_int
    L.sv_sample_rows.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, vp,
                                 ctypes.c_int64, vp, ctypes.c_int64, vp, vp, ctypes.c_uint64,
                                 ctypes.c_uint32, ctypes.c_uint32, vp, ctypes.c_int64, vp]
    L.sv_sample_rows.restype = ctypes.c_int
    L.sv_verify_batch_sharded.argtypes = [ctypes.POINTER(SvVerifyArgs), ctypes.c_int32,
                                          ctypes.c_int64, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                          vp]
    L.sv_verify_batch_sharded.restype = ctypes.c_int
    L.sv_stream_read.argtypes = [vp, ctypes.c_size_t, ctypes.c_int32, vp, vp]
    L.sv_stream_read.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().sv_status_string(status).decode()


def _check(status: int, what: str):
    if status != SV_OK:
        raise SpecVerifyError(f"{what}: {status_string(status)} (status {status})")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def k_rho(B: int, D: int, rho: float) -> int:
    return int(load().sv_k_rho(B, D, rho))


def workspace_bytes(B: int, D_max: int, V: int) -> int:
    return int(load().sv_verify_workspace_bytes(B, D_max, V))


def _rows_view(t: torch.Tensor) -> tuple[torch.Tensor, int]:
    """A logits tensor as rows of V elements: returns (tensor, row stride)."""
    if t.dim() == 2:
        if t.stride(1) != 1:
            raise ValueError("logits rows must be contiguous")
        return t, t.stride(0)
    t2 = t.reshape(-1, t.shape[-1])
    if t2.data_ptr() != t.data_ptr() or t2.stride(1) != 1:
        raise ValueError("logits must reshape to (rows, V) without a copy")
    return t2, t2.stride(0)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return SV_DTYPE_BF16
    if dt == torch.float32:
        return SV_DTYPE_FP32
    raise ValueError(f"unsupported logits dtype {dt}")


def allocate_budget(conf: torch.Tensor, K: int, max_depth: torch.Tensor | None = None,
                    out: dict | None = None) -> dict:
    """D-cut budget on the GPU.  conf: float32 (B, D_max) device tensor."""
    assert conf.is_cuda and conf.dtype == torch.float32 and conf.is_contiguous()
    B, D = conf.shape
    dev = conf.device
    if out is None:
        out = dict(depth=torch.empty(B, dtype=torch.int32, device=dev),
                   draft_row0=torch.empty(B, dtype=torch.int64, device=dev),
                   target_row0=torch.empty(B, dtype=torch.int64, device=dev),
                   utility=torch.empty(2, dtype=torch.float32, device=dev))
    md = None
    if max_depth is not None:
        md = max_depth.to(device=dev, dtype=torch.int32).contiguous()
    st = load().sv_allocate_budget(_ptr(conf), B, D, _ptr(md), int(K), _ptr(out["depth"]),
                                   _ptr(out["draft_row0"]), _ptr(out["target_row0"]),
                                   _ptr(out["utility"]), _stream(dev))
    _check(st, "sv_allocate_budget")
    return out


def allocate_fixed_depth(conf: torch.Tensor, K: int, out: dict | None = None) -> dict:
    """The fixed-depth baseline on the GPU (sv_allocate_fixed_depth): the same
    outputs as allocate_budget.  conf: float32 (B, D_max) device tensor."""
    assert conf.is_cuda and conf.dtype == torch.float32 and conf.is_contiguous()
    B, D = conf.shape
    dev = conf.device
    if out is None:
        out = dict(depth=torch.empty(B, dtype=torch.int32, device=dev),
                   draft_row0=torch.empty(B, dtype=torch.int64, device=dev),
                   target_row0=torch.empty(B, dtype=torch.int64, device=dev),
                   utility=torch.empty(2, dtype=torch.float32, device=dev))
    st = load().sv_allocate_fixed_depth(_ptr(conf), B, D, int(K), _ptr(out["depth"]),
                                        _ptr(out["draft_row0"]), _ptr(out["target_row0"]),
                                        _ptr(out["utility"]), _stream(dev))
    _check(st, "sv_allocate_fixed_depth")
    return out


class DraftConfidence:
    """The drafter's confidence q_k(d_k) of every drafted token, computed on
    the GPU from the draft rows (sv_draft_confidence).  Holds its workspace."""

    def __init__(self, B: int, D_max: int, V: int, dtype: torch.dtype, device):
        self.B, self.D, self.V = B, D_max, V
        self.device = torch.device(device)
        self.code = _dtype_code(dtype)
        nbytes = int(load().sv_draft_confidence_workspace_bytes(self.code, B, D_max, V))
        if nbytes == 0:
            raise ValueError("sv_draft_confidence: unsupported sizes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.conf = torch.empty((B, D_max), dtype=torch.float32, device=self.device)

    def __call__(self, draft: torch.Tensor, draft_row0: torch.Tensor, draft_tokens: torch.Tensor,
                 temperature: torch.Tensor, depth: torch.Tensor | None = None) -> torch.Tensor:
        rows, stride = _rows_view(draft)
        if rows.shape[-1] != self.V or _dtype_code(rows.dtype) != self.code:
            raise ValueError("draft logits do not match the sizes this object was built for")
        dr0 = draft_row0.to(device=self.device, dtype=torch.int64).contiguous()
        tok = draft_tokens.to(device=self.device, dtype=torch.int32).contiguous()
        T = temperature.to(device=self.device, dtype=torch.float32).contiguous()
        dep = None if depth is None else depth.to(device=self.device, dtype=torch.int32).contiguous()
        self._keep = (dr0, tok, T, dep)
        st = load().sv_draft_confidence(self.code, self.B, self.D, self.V, stride, _ptr(rows),
                                        _ptr(dr0), _ptr(tok), _ptr(dep), _ptr(T), _ptr(self.conf),
                                        _ptr(self.workspace), self.workspace.numel(),
                                        _stream(self.device))
        _check(st, "sv_draft_confidence")
        return self.conf


def draft_confidence(draft, draft_row0, draft_tokens, temperature, depth=None) -> torch.Tensor:
    B, D = draft_tokens.shape
    return DraftConfidence(B, D, draft.shape[-1], draft.dtype, draft.device)(
        draft, draft_row0, draft_tokens, temperature, depth).clone()


def select_budget_ratio(conf: torch.Tensor, table_batch, table_latency, ratios=DCUT_RATIOS,
                        max_depth: torch.Tensor | None = None) -> dict:
    """D-cut keep-ratio choice on the GPU, then the budget at the chosen K.
    table_latency: (len(table_batch), len(ratios)) latencies (host values)."""
    assert conf.is_cuda and conf.dtype == torch.float32 and conf.is_contiguous()
    B, D = conf.shape
    dev = conf.device
    rr = [float(x) for x in ratios]
    tb = [int(x) for x in table_batch]
    tl = [float(x) for row in table_latency for x in row]
    if len(tl) != len(tb) * len(rr):
        raise ValueError("table_latency must have one row per batch size and one column per ratio")
    c_r = (ctypes.c_double * len(rr))(*rr)
    c_b = (ctypes.c_int32 * len(tb))(*tb)
    c_l = (ctypes.c_float * len(tl))(*tl)
    out = dict(choice=torch.empty(1, dtype=torch.int32, device=dev),
               K=torch.empty(1, dtype=torch.int64, device=dev),
               projected=torch.empty(len(rr), dtype=torch.float32, device=dev),
               depth=torch.empty(B, dtype=torch.int32, device=dev),
               draft_row0=torch.empty(B, dtype=torch.int64, device=dev),
               target_row0=torch.empty(B, dtype=torch.int64, device=dev),
               utility=torch.empty(2, dtype=torch.float32, device=dev))
    md = None if max_depth is None else max_depth.to(device=dev, dtype=torch.int32).contiguous()
    st = load().sv_select_budget_ratio(_ptr(conf), B, D, _ptr(md), len(rr), c_r, len(tb), c_b, c_l,
                                       _ptr(out["choice"]), _ptr(out["K"]), _ptr(out["projected"]),
                                       _ptr(out["depth"]), _ptr(out["draft_row0"]),
                                       _ptr(out["target_row0"]), _ptr(out["utility"]),
                                       _stream(dev))
    _check(st, "sv_select_budget_ratio")
    return out


def sample_rows(logits: torch.Tensor, row_index: torch.Tensor, temperature: torch.Tensor,
                tokens: torch.Tensor, *, seed: int = 0, step: int = 0, position: int = 0,
                request_id: torch.Tensor | None = None, row_base: int = 0) -> torch.Tensor:
    """One token per request from softmax(row / T) on the verifier's Philox
    stream (sv_sample_rows).  row_index and tokens are int32 device tensors of
    B entries (any stride: a column of a (B, D) matrix works); logits is
    (rows, V) with contiguous rows."""
    rows, stride = _rows_view(logits)
    B = tokens.shape[0]
    assert row_index.dtype == torch.int32 and tokens.dtype == torch.int32
    assert row_index.shape[0] == B and temperature.shape[0] == B
    T = temperature.to(dtype=torch.float32).contiguous()
    rid = None if request_id is None else request_id.to(dtype=torch.int32).contiguous()
    st = load().sv_sample_rows(_dtype_code(rows.dtype), B, rows.shape[-1], stride, _ptr(rows),
                               int(row_base), _ptr(row_index), row_index.stride(0), _ptr(T),
                               _ptr(rid), int(seed), int(step), int(position), _ptr(tokens),
                               tokens.stride(0), _stream(rows.device))
    _check(st, "sv_sample_rows")
    return tokens


@dataclass
class VerifyOutputs:
    accepted_len: torch.Tensor
    out_tokens: torch.Tensor
    num_out: torch.Tensor
    alpha: torch.Tensor | None
    diag: torch.Tensor | None  # (B, 4) int32 view of sv_diag: margins as float bits, bits
    # acceptance statistics of the batch, as accept_stats returns them, or None
    stats: dict | None = None

    def margins(self):
        d = self.diag.view(torch.float32)
        return d[:, 0], d[:, 1]

    def bits(self):
        return self.diag[:, 2]


class Verifier:
    """Holds the output buffers, the workspace and a prepared argument block
    for repeated verification of batches with the same shapes."""

    def __init__(self, B: int, D_max: int, V: int, device, alpha: bool = True,
                 diag: bool = True, stats: bool = False):
        """stats=True asks the call for the batch's acceptance statistics
        (the stats_* outputs of sv_verify_args, the bits of accept_stats on
        the call's depth, alpha and accepted lengths) in out.stats."""
        self.B, self.D_max, self.V = B, D_max, V
        self.device = torch.device(device)
        dev = self.device
        self.out = VerifyOutputs(
            accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
            out_tokens=torch.empty((B, D_max + 1), dtype=torch.int32, device=dev),
            num_out=torch.empty(B, dtype=torch.int32, device=dev),
            alpha=torch.empty((B, D_max), dtype=torch.float32, device=dev) if alpha else None,
            diag=torch.empty((B, 4), dtype=torch.int32, device=dev) if diag else None,
            stats=dict(expected_len=torch.empty(B, dtype=torch.float32, device=dev),
                       per_depth=torch.empty(3 * max(D_max, 1), dtype=torch.float32, device=dev),
                       summary=torch.empty(4, dtype=torch.float32, device=dev))
            if stats else None)
        self.ws_bytes = workspace_bytes(B, D_max, V)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.args = SvVerifyArgs()
        self._keep = []
        self._shards = None

    def prepare(self, target, draft, target_row0, draft_row0, draft_tokens, depth, temperature,
                *, seed: int = 0, step: int = 0, request_id=None, flags: int = 0,
                _shard: bool = False):
        """Fill the argument block; the tensors must stay alive while used."""
        tgt, stride = _rows_view(target)
        if tgt.shape[1] < self.V and not _shard:
            raise ValueError("row width below V")
        self._shards = None
        a = self.args
        a.dtype = _dtype_code(tgt.dtype)
        a.B, a.D_max, a.V, a.row_stride = self.B, self.D_max, self.V, stride
        a.target_logits = tgt.data_ptr()
        a.target_row0 = target_row0.data_ptr()
        if draft is not None:
            dft, dstride = _rows_view(draft)
            if dstride != stride or dft.dtype != tgt.dtype:
                raise ValueError("target and draft logits need the same dtype and row stride")
            a.draft_logits = dft.data_ptr()
            a.draft_row0 = draft_row0.data_ptr()
        else:
            a.draft_logits = None
            a.draft_row0 = None
        a.draft_tokens = draft_tokens.data_ptr() if draft_tokens is not None else None
        a.depth = depth.data_ptr()
        a.temperature = temperature.data_ptr()
        a.request_id = request_id.data_ptr() if request_id is not None else None
        a.seed, a.step, a.flags = int(seed), int(step), int(flags)
        o = self.out
        a.accepted_len = o.accepted_len.data_ptr()
        a.out_tokens = o.out_tokens.data_ptr()
        a.num_out = o.num_out.data_ptr()
        a.alpha = _ptr(o.alpha) if o.alpha is not None and o.alpha.numel() else None
        a.diag = _ptr(o.diag)
        if o.stats is not None:
            a.stats_expected_len = _ptr(o.stats["expected_len"])
            a.stats_per_depth = _ptr(o.stats["per_depth"])
            a.stats_summary = _ptr(o.stats["summary"])
        else:
            a.stats_expected_len = a.stats_per_depth = a.stats_summary = None
        a.workspace = self.workspace.data_ptr()
        a.workspace_bytes = self.workspace.numel()
        self._keep = [target, draft, target_row0, draft_row0, draft_tokens, depth, temperature,
                      request_id]
        return self

    def prepare_sharded(self, target_shards, draft_shards, shard_width: int, target_row0,
                        draft_row0, draft_tokens, depth, temperature, *, seed: int = 0,
                        step: int = 0, request_id=None, flags: int = 0):
        """Like prepare, for logits split over vocabulary shards: shard s of a
        row holds columns [s W, min(V, (s + 1) W)); every shard a (rows, width)
        tensor with the same contiguous-row stride (sv_verify_batch_sharded)."""
        views = [_rows_view(t) for t in target_shards]
        stride = views[0][1]
        if any(st != stride for _, st in views):
            raise ValueError("every shard needs the same row stride")
        self.prepare(views[0][0], None if draft_shards is None else _rows_view(draft_shards[0])[0],
                     target_row0, draft_row0, draft_tokens, depth, temperature, seed=seed,
                     step=step, request_id=request_id, flags=flags, _shard=True)
        self.args.row_stride = stride
        self.args.target_logits = None
        self.args.draft_logits = None
        n = len(target_shards)
        self._tsh = (ctypes.c_void_p * n)(*[t.data_ptr() for t, _ in views])
        self._dsh = None
        if draft_shards is not None:
            dv = [_rows_view(t) for t in draft_shards]
            if any(st != stride for _, st in dv) or len(dv) != n:
                raise ValueError("draft shards must match the target shards")
            self._dsh = (ctypes.c_void_p * n)(*[t.data_ptr() for t, _ in dv])
        self._shards = (n, int(shard_width))
        self._keep.append((target_shards, draft_shards))
        return self

    def set_stage_events(self, events):
        """Ask for SV_NUM_STAGE_EVENTS torch.cuda.Event objects (timing
        enabled; an entry may be None) to be recorded at the stage
        boundaries; None switches off."""
        if events is None:
            self.args.stage_events = None
            self._events = None
            return
        assert len(events) == SV_NUM_STAGE_EVENTS
        for e in events:  # torch creates the HIP event on first record
            if e is not None and e.cuda_event == 0:
                e.record()
        self._events = (ctypes.c_void_p * SV_NUM_STAGE_EVENTS)(
            *[e.cuda_event if e is not None else None for e in events])
        self.args.stage_events = ctypes.cast(self._events, ctypes.c_void_p)

    def run(self, noalloc: bool = False) -> VerifyOutputs:
        """One verification call; noalloc=True calls sv_verify_batch_noalloc
        (the library's static scratch instead of this object's workspace)."""
        if noalloc:
            if self._shards is not None:
                raise ValueError("the no-allocation entry point takes unsharded logits")
            st = load().sv_verify_batch_noalloc(ctypes.byref(self.args), _stream(self.device))
            _check(st, "sv_verify_batch_noalloc")
            return self.out
        if self._shards is not None:
            n, w = self._shards
            st = load().sv_verify_batch_sharded(ctypes.byref(self.args), n, w, self._tsh,
                                                self._dsh, _stream(self.device))
            _check(st, "sv_verify_batch_sharded")
            return self.out
        st = load().sv_verify_batch(ctypes.byref(self.args), _stream(self.device))
        _check(st, "sv_verify_batch")
        return self.out


def verify(target: torch.Tensor, draft: torch.Tensor | None, target_row0: torch.Tensor,
           draft_row0: torch.Tensor | None, draft_tokens: torch.Tensor, depth: torch.Tensor,
           temperature: torch.Tensor, *, V: int | None = None, seed: int = 0, step: int = 0,
           request_id: torch.Tensor | None = None, alpha: bool = True, diag: bool = True,
           flags: int = 0) -> VerifyOutputs:
    """One call of sv_verify_batch with freshly allocated outputs."""
    B = depth.numel()
    D_max = draft_tokens.shape[1] if draft_tokens is not None and draft_tokens.dim() == 2 else 0
    V = target.shape[-1] if V is None else V
    v = Verifier(B, D_max, V, target.device, alpha=alpha, diag=diag)
    v.prepare(target, draft, target_row0, draft_row0, draft_tokens, depth, temperature, seed=seed,
              step=step, request_id=request_id, flags=flags)
    return v.run()


def stream_read(buf: torch.Tensor, sink: torch.Tensor, blocks_per_cu: int = 4) -> None:
    """Calibration: one plain streaming read of buf (sv_stream_read)."""
    assert buf.is_cuda and buf.is_contiguous() and sink.is_cuda and sink.numel() >= 1
    nbytes = buf.numel() * buf.element_size() // 16 * 16
    st = load().sv_stream_read(_ptr(buf), nbytes, int(blocks_per_cu), _ptr(sink),
                               _stream(buf.device))
    _check(st, "sv_stream_read")


def accept_stats(depth: torch.Tensor, alpha: torch.Tensor | None, accepted_len: torch.Tensor,
                 D_max: int) -> dict:
    B = depth.numel()
    dev = depth.device
    out = dict(expected_len=torch.empty(B, dtype=torch.float32, device=dev),
               per_depth=torch.empty(3 * max(D_max, 1), dtype=torch.float32, device=dev),
               summary=torch.empty(4, dtype=torch.float32, device=dev))
    st = load().sv_accept_stats(_ptr(depth), _ptr(alpha), _ptr(accepted_len), B, D_max,
                                _ptr(out["expected_len"]), _ptr(out["per_depth"]),
                                _ptr(out["summary"]), _stream(dev))
    _check(st, "sv_accept_stats")
    return out


class AcceptAccumulator:
    """Running acceptance statistics over verified batches
    (sv_accept_stats_accumulate): totals on the device, summary =
    (MAL, expected MAL, mean acceptance, P(tau >= 1..D_max))."""

    def __init__(self, D_max: int, device):
        self.D = D_max
        self.accum = torch.zeros(3 + 2 * D_max, dtype=torch.float64, device=device)
        self.summary = torch.zeros(3 + D_max, dtype=torch.float32, device=device)

    def add(self, depth: torch.Tensor, alpha: torch.Tensor | None, accepted_len: torch.Tensor):
        st = load().sv_accept_stats_accumulate(_ptr(depth), _ptr(alpha), _ptr(accepted_len),
                                               depth.numel(), self.D, _ptr(self.accum),
                                               _ptr(self.summary), _stream(depth.device))
        _check(st, "sv_accept_stats_accumulate")
        return self.summary
