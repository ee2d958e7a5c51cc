"""CPU oracle for batched lossless draft verification and the verification budget.

TEST INFRASTRUCTURE ONLY.  The oracle is the plain, slow, single-threaded C
statement of the method (``svo.c``); this module builds it with gcc and wraps
it with ctypes over numpy arrays.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it.  It shares no code with the HIP
library and the HIP library never calls it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "svo.c")
LIB_PATH = os.path.join(_HERE, "libsvo.so")

# Flags: no fast-math, no FMA contraction, IEEE float32 on SSE.
GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-Wall", "-Wextra", "-Werror"]

BIT_BAD_DEPTH = 1
BIT_BAD_TOKEN = 2
BIT_BAD_ROW = 4
BIT_RESIDUAL_ZERO = 8
BIT_BAD_TEMPERATURE = 16


def build() -> str:
    """Compile ``svo.c`` into ``libsvo.so`` next to it; returns the path."""
    tmp = LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, SOURCE, "-lm"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u32p = ctypes.POINTER(ctypes.c_uint32)


def lib() -> ctypes.CDLL:
    """Load the oracle library, building it first if it is missing or stale."""
    global _lib
    if _lib is not None:
        return _lib
    if (not os.path.exists(LIB_PATH)
            or os.path.getmtime(LIB_PATH) < max(os.path.getmtime(SOURCE),
                                                 os.path.getmtime(os.path.join(_HERE, "svo.h")))):
        build()
    L = ctypes.CDLL(LIB_PATH)
    L.svo_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
    L.svo_philox4x32_10.restype = None
    L.svo_u24.argtypes = [ctypes.c_uint32]
    L.svo_u24.restype = ctypes.c_double
    L.svo_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                               _f64p, _f64p]
    L.svo_uniforms.restype = None
    L.svo_row_valid.argtypes = [_f32p, ctypes.c_int64]
    L.svo_row_valid.restype = ctypes.c_int
    L.svo_argmax.argtypes = [_f32p, ctypes.c_int64]
    L.svo_argmax.restype = ctypes.c_int64
    L.svo_log_normalizer.argtypes = [_f32p, ctypes.c_int64, ctypes.c_double]
    L.svo_log_normalizer.restype = ctypes.c_double
    L.svo_prob.argtypes = [_f32p, ctypes.c_int64, ctypes.c_double, ctypes.c_int64]
    L.svo_prob.restype = ctypes.c_double
    L.svo_alpha.argtypes = [_f32p, _f32p, ctypes.c_int64, ctypes.c_double]
    L.svo_alpha.restype = ctypes.c_double
    L.svo_accept.argtypes = [_f32p, _f32p, ctypes.c_int64, ctypes.c_double, ctypes.c_int32,
                             ctypes.c_double, _f64p]
    L.svo_accept.restype = ctypes.c_int
    L.svo_sample_residual.argtypes = [_f32p, _f32p, ctypes.c_int64, ctypes.c_double,
                                      ctypes.c_double, _f64p, _f64p]
    L.svo_sample_residual.restype = ctypes.c_int64
    L.svo_sample_target.argtypes = [_f32p, ctypes.c_int64, ctypes.c_double, ctypes.c_double, _f64p]
    L.svo_sample_target.restype = ctypes.c_int64
    L.svo_expected_accepted.argtypes = [_f64p, ctypes.c_int32]
    L.svo_expected_accepted.restype = ctypes.c_double
    L.svo_verify_request.argtypes = [ctypes.POINTER(_f32p), ctypes.POINTER(_f32p), _i32p,
                                     ctypes.c_int32, ctypes.c_int64, ctypes.c_float, _f64p, _f64p,
                                     _i32p, _f64p, _f64p, _u32p]
    L.svo_verify_request.restype = ctypes.c_int32
    L.svo_verify_batch.argtypes = [_f32p, _f32p, ctypes.c_int64, ctypes.c_int64, _i64p, _i64p,
                                   _i32p, _i32p, _f32p, _u32p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_uint64, ctypes.c_uint32, _i32p, _i32p, _i32p, _f64p,
                                   _f64p, _f64p, _u32p, _i32p]
    L.svo_verify_batch.restype = ctypes.c_int
    L.svo_k_rho.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_double]
    L.svo_k_rho.restype = ctypes.c_int64
    L.svo_allocate_budget.argtypes = [_f32p, ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int64,
                                      _i32p, _i64p, _i64p, _f64p]
    L.svo_allocate_budget.restype = ctypes.c_int
    L.svo_fixed_depth.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, _i32p]
    L.svo_fixed_depth.restype = None
    L.svo_fixed_depth_budget.argtypes = [_f32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                         _i32p, _i64p, _i64p, _f64p]
    L.svo_fixed_depth_budget.restype = ctypes.c_int
    L.svo_accept_stats.argtypes = [_i32p, _f64p, _i32p, ctypes.c_int32, ctypes.c_int32, _f64p,
                                   _f64p, _f64p]
    L.svo_accept_stats.restype = ctypes.c_int
    L.svo_accept_accumulate.argtypes = [_i32p, _f64p, _i32p, ctypes.c_int32, ctypes.c_int32,
                                        _f64p, _f64p]
    L.svo_accept_accumulate.restype = ctypes.c_int
    L.svo_draft_confidence.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int32, _i64p, _i32p, _i32p, _f32p, _f32p]
    L.svo_draft_confidence.restype = ctypes.c_int
    L.svo_table_latency.argtypes = [ctypes.c_int32, _i32p, _f32p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32]
    L.svo_table_latency.restype = ctypes.c_double
    L.svo_select_budget_ratio.argtypes = [_f32p, ctypes.c_int32, ctypes.c_int32, _i32p,
                                          ctypes.c_int32, _f64p, ctypes.c_int32, _i32p, _f32p,
                                          _i32p, _i64p, _f64p, _i32p, _i64p, _i64p, _f64p]
    L.svo_select_budget_ratio.restype = ctypes.c_int
    _lib = L
    return L


def _p(a: np.ndarray | None, ptype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ptype)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# ---- random numbers --------------------------------------------------------

def philox(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().svo_philox4x32_10(_p(c, _u32p), _p(k, _u32p), _p(out, _u32p))
    return out


def u24(w: int) -> float:
    return lib().svo_u24(int(w) & 0xFFFFFFFF)


def uniforms(seed: int, request_id: int, step: int, position: int) -> tuple[float, float]:
    a = ctypes.c_double()
    s = ctypes.c_double()
    lib().svo_uniforms(seed, request_id, step, position, ctypes.byref(a), ctypes.byref(s))
    return a.value, s.value


# ---- one row ---------------------------------------------------------------

def row_valid(x) -> bool:
    x = _f32(x)
    return bool(lib().svo_row_valid(_p(x, _f32p), x.size))


def argmax(x) -> int:
    x = _f32(x)
    return int(lib().svo_argmax(_p(x, _f32p), x.size))


def log_normalizer(x, T: float) -> float:
    x = _f32(x)
    return lib().svo_log_normalizer(_p(x, _f32p), x.size, float(T))


def prob(x, T: float, y: int) -> float:
    x = _f32(x)
    return lib().svo_prob(_p(x, _f32p), x.size, float(T), int(y))


def alpha(P, Q, T: float) -> float:
    P, Q = _f32(P), _f32(Q)
    return lib().svo_alpha(_p(P, _f32p), _p(Q, _f32p), P.size, float(T))


def accept(P, Q, T: float, d: int, u: float) -> tuple[bool, float]:
    P, Q = _f32(P), _f32(Q)
    r = ctypes.c_double()
    k = lib().svo_accept(_p(P, _f32p), _p(Q, _f32p), P.size, float(T), int(d), float(u),
                         ctypes.byref(r))
    return bool(k), r.value


def sample_residual(P, Q, T: float, u: float) -> tuple[int, float, float]:
    P, Q = _f32(P), _f32(Q)
    m = ctypes.c_double()
    R = ctypes.c_double()
    y = lib().svo_sample_residual(_p(P, _f32p), _p(Q, _f32p), P.size, float(T), float(u),
                                  ctypes.byref(m), ctypes.byref(R))
    return int(y), m.value, R.value


def sample_target(P, T: float, u: float) -> tuple[int, float]:
    P = _f32(P)
    m = ctypes.c_double()
    y = lib().svo_sample_target(_p(P, _f32p), P.size, float(T), float(u), ctypes.byref(m))
    return int(y), m.value


def expected_accepted(alpha_vec) -> float:
    a = np.ascontiguousarray(alpha_vec, dtype=np.float64)
    return lib().svo_expected_accepted(_p(a, _f64p), a.size)


# ---- one request with explicit uniforms -------------------------------------

def verify_request(P_rows, Q_rows, d, T: float, u_accept, u_sample):
    """P_rows: (n+1, V) float32, Q_rows: (n, V) or None, d: (n,) draft tokens.
    Returns (tau, emitted tokens, accept_margin, draw_margin, bits)."""
    P_rows = _f32(P_rows)
    n = P_rows.shape[0] - 1
    V = P_rows.shape[1]
    Pp = (_f32p * (n + 1))(*[P_rows[k].ctypes.data_as(_f32p) for k in range(n + 1)])
    if Q_rows is not None:
        Q_rows = _f32(Q_rows)
        Qp = (_f32p * max(n, 1))(*[Q_rows[k].ctypes.data_as(_f32p) for k in range(n)])
    else:
        Qp = (_f32p * max(n, 1))()
    dd = np.ascontiguousarray(d, dtype=np.int32).reshape(-1)
    if dd.size == 0:
        dd = np.zeros(1, dtype=np.int32)
    ua = np.ascontiguousarray(u_accept, dtype=np.float64).reshape(-1)
    if ua.size == 0:
        ua = np.zeros(1)
    us = np.ascontiguousarray(u_sample, dtype=np.float64)
    out = np.full(n + 1, -1, dtype=np.int32)
    am = ctypes.c_double()
    dm = ctypes.c_double()
    bits = ctypes.c_uint32(0)
    tau = lib().svo_verify_request(Pp, Qp, _p(dd, _i32p), n, V, ctypes.c_float(T),
                                   _p(ua, _f64p), _p(us, _f64p), _p(out, _i32p),
                                   ctypes.byref(am), ctypes.byref(dm), ctypes.byref(bits))
    return int(tau), out[: tau + 1].copy(), am.value, dm.value, bits.value


# ---- the batch ------------------------------------------------------------

def verify_batch(target, draft, target_row0, draft_row0, draft_tokens, depth, temperature,
                 seed: int = 0, step: int = 0, request_id=None, D_max: int | None = None):
    """target: (rows, V) float32 host array; draft: (rows, V) or None.
    Returns a dict of numpy arrays (accepted_len, out_tokens, num_out, alpha,
    accept_margin, draw_margin, bits, draws)."""
    target = _f32(target)
    V = target.shape[-1]
    target = target.reshape(-1, V)
    draft_arr = None if draft is None else _f32(draft).reshape(-1, V)
    tr0 = np.ascontiguousarray(target_row0, dtype=np.int64)
    B = tr0.size
    dr0 = np.ascontiguousarray(draft_row0 if draft_row0 is not None else np.zeros(B),
                               dtype=np.int64)
    tok = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    if D_max is None:
        D_max = tok.shape[1] if tok.ndim == 2 else 0
    tok = tok.reshape(B, D_max) if B * D_max > 0 else np.zeros((max(B, 1), max(D_max, 1)),
                                                                  dtype=np.int32)
    dep = np.ascontiguousarray(depth, dtype=np.int32)
    temp = np.ascontiguousarray(temperature, dtype=np.float32)
    rid = None if request_id is None else np.ascontiguousarray(request_id, dtype=np.uint32)
    acc = np.zeros(B, dtype=np.int32)
    out = np.zeros((B, D_max + 1), dtype=np.int32)
    num = np.zeros(B, dtype=np.int32)
    al = np.zeros((B, max(D_max, 1)), dtype=np.float64)
    am = np.zeros(B, dtype=np.float64)
    dm = np.zeros(B, dtype=np.float64)
    bits = np.zeros(B, dtype=np.uint32)
    draws = np.zeros(B, dtype=np.int32)
    st = lib().svo_verify_batch(_p(target, _f32p), _p(draft_arr, _f32p), V, V, _p(tr0, _i64p),
                                _p(dr0, _i64p), _p(tok, _i32p), _p(dep, _i32p), _p(temp, _f32p),
                                _p(rid, _u32p), B, D_max, seed, step, _p(acc, _i32p),
                                _p(out, _i32p), _p(num, _i32p), _p(al, _f64p), _p(am, _f64p),
                                _p(dm, _f64p), _p(bits, _u32p), _p(draws, _i32p))
    if st != 0:
        raise ValueError(f"svo_verify_batch: invalid argument (status {st})")
    return dict(accepted_len=acc, out_tokens=out, num_out=num, alpha=al[:, :D_max],
                accept_margin=am, draw_margin=dm, bits=bits, draws=draws)


# ---- budget ----------------------------------------------------------------

def k_rho(B: int, D: int, rho: float) -> int:
    return int(lib().svo_k_rho(B, D, rho))


def allocate_budget(conf, K: int, max_depth=None):
    c = _f32(conf)
    B, D = c.shape
    md = None if max_depth is None else np.ascontiguousarray(max_depth, dtype=np.int32)
    depth = np.zeros(B, dtype=np.int32)
    dr0 = np.zeros(B, dtype=np.int64)
    tr0 = np.zeros(B, dtype=np.int64)
    util = np.zeros(2, dtype=np.float64)
    st = lib().svo_allocate_budget(_p(c, _f32p), B, D, _p(md, _i32p), int(K), _p(depth, _i32p),
                                   _p(dr0, _i64p), _p(tr0, _i64p), _p(util, _f64p))
    if st != 0:
        raise ValueError("svo_allocate_budget: invalid argument")
    return dict(depth=depth, draft_row0=dr0, target_row0=tr0, utility=util)


def fixed_depth(B: int, D: int, K: int) -> np.ndarray:
    depth = np.zeros(B, dtype=np.int32)
    lib().svo_fixed_depth(B, D, int(K), _p(depth, _i32p))
    return depth


def fixed_depth_budget(conf, K: int):
    """The fixed-depth baseline at K: depths, row offsets and utility
    (kept products, all products), as allocate_budget returns them."""
    c = _f32(conf)
    B, D = c.shape
    depth = np.zeros(B, dtype=np.int32)
    dr0 = np.zeros(B, dtype=np.int64)
    tr0 = np.zeros(B, dtype=np.int64)
    util = np.zeros(2, dtype=np.float64)
    st = lib().svo_fixed_depth_budget(_p(c, _f32p), B, D, int(K), _p(depth, _i32p),
                                      _p(dr0, _i64p), _p(tr0, _i64p), _p(util, _f64p))
    if st != 0:
        raise ValueError("svo_fixed_depth_budget: invalid argument")
    return dict(depth=depth, draft_row0=dr0, target_row0=tr0, utility=util)


# ---- drafter confidence and keep-ratio choice --------------------------------

def draft_confidence(draft, draft_row0, draft_tokens, temperature, depth=None):
    """conf[r, k] = softmax(draft row draft_row0[r] + k / T_r)[d_rk] (T = 0 read as 1)
    for k < depth[r]; 0 past the depth; NaN for invalid rows, tokens, depths or
    temperatures.  draft: (rows, V) float32; draft_tokens: (B, D_max) int32."""
    x = _f32(draft)
    V = x.shape[1]
    tok = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    B, D = tok.shape
    dr0 = np.ascontiguousarray(draft_row0, dtype=np.int64)
    T = np.ascontiguousarray(temperature, dtype=np.float32)
    dep = None if depth is None else np.ascontiguousarray(depth, dtype=np.int32)
    conf = np.zeros((B, D), dtype=np.float32)
    st = lib().svo_draft_confidence(_p(x, _f32p), V, V, B, D, _p(dr0, _i64p), _p(tok, _i32p),
                                    _p(dep, _i32p), _p(T, _f32p), _p(conf, _f32p))
    if st != 0:
        raise ValueError("svo_draft_confidence: invalid argument")
    return conf


def table_latency(table_batch, table_latency_rows, j: int, B: int) -> float:
    tb = np.ascontiguousarray(table_batch, dtype=np.int32)
    tl = np.ascontiguousarray(table_latency_rows, dtype=np.float32)
    return lib().svo_table_latency(tb.size, _p(tb, _i32p), _p(tl, _f32p), tl.shape[1], int(j), int(B))


def select_budget_ratio(conf, ratios, table_batch, table_latency_rows, max_depth=None):
    """D-cut keep-ratio choice.  table_latency_rows: (n_batch, n_ratios)."""
    c = _f32(conf)
    B, D = c.shape
    rr = np.ascontiguousarray(ratios, dtype=np.float64)
    tb = np.ascontiguousarray(table_batch, dtype=np.int32)
    tl = np.ascontiguousarray(table_latency_rows, dtype=np.float32)
    md = None if max_depth is None else np.ascontiguousarray(max_depth, dtype=np.int32)
    choice = np.zeros(1, dtype=np.int32)
    K = np.zeros(1, dtype=np.int64)
    proj = np.zeros(rr.size, dtype=np.float64)
    depth = np.zeros(B, dtype=np.int32)
    dr0 = np.zeros(B, dtype=np.int64)
    tr0 = np.zeros(B, dtype=np.int64)
    util = np.zeros(2, dtype=np.float64)
    st = lib().svo_select_budget_ratio(_p(c, _f32p), B, D, _p(md, _i32p), rr.size, _p(rr, _f64p),
                                       tb.size, _p(tb, _i32p), _p(tl, _f32p), _p(choice, _i32p),
                                       _p(K, _i64p), _p(proj, _f64p), _p(depth, _i32p),
                                       _p(dr0, _i64p), _p(tr0, _i64p), _p(util, _f64p))
    if st != 0:
        raise ValueError("svo_select_budget_ratio: invalid argument")
    return dict(choice=int(choice[0]), K=int(K[0]), projected=proj, depth=depth, draft_row0=dr0,
                target_row0=tr0, utility=util)


# ---- statistics ------------------------------------------------------------

def accept_stats(depth, alpha_mat, accepted_len, D_max: int):
    dep = np.ascontiguousarray(depth, dtype=np.int32)
    B = dep.size
    al = None if alpha_mat is None else np.ascontiguousarray(alpha_mat, dtype=np.float64).reshape(
        B, D_max)
    acc = np.ascontiguousarray(accepted_len, dtype=np.int32)
    e = np.zeros(B, dtype=np.float64)
    pd = np.zeros(3 * max(D_max, 1), dtype=np.float64)
    sm = np.zeros(4, dtype=np.float64)
    st = lib().svo_accept_stats(_p(dep, _i32p), _p(al, _f64p), _p(acc, _i32p), B, D_max,
                                _p(e, _f64p), _p(pd, _f64p), _p(sm, _f64p))
    if st != 0:
        raise ValueError("svo_accept_stats: invalid argument")
    return dict(expected_len=e, per_depth=pd[: 3 * D_max].reshape(3, D_max), summary=sm)


def accept_accumulate(depth, alpha_mat, accepted_len, D_max: int, accum=None):
    """Adds one verified batch to the running statistics accum (a float64
    array of 3 + 2 D_max, created when None); returns (accum, summary) with
    summary = (MAL, expected MAL, mean acceptance, P(tau >= 1..D_max))."""
    dep = np.ascontiguousarray(depth, dtype=np.int32)
    B = dep.size
    al = None if alpha_mat is None else np.ascontiguousarray(alpha_mat, dtype=np.float64).reshape(
        B, D_max)
    acc = np.ascontiguousarray(accepted_len, dtype=np.int32)
    if accum is None:
        accum = np.zeros(3 + 2 * D_max, dtype=np.float64)
    summ = np.zeros(3 + D_max, dtype=np.float64)
    st = lib().svo_accept_accumulate(_p(dep, _i32p), _p(al, _f64p), _p(acc, _i32p), B, D_max,
                                     _p(accum, _f64p), _p(summ, _f64p))
    if st != 0:
        raise ValueError("svo_accept_accumulate: invalid argument")
    return accum, summ


# ---- multi-step decoding on a Markov target ---------------------------------
# The decode loop the pages' eval server runs ([T] "The MTP path": MAL and
# position-wise acceptance measured over whole generations; [A] "MTP": a
# block of drafts is verified in one target pass and one rejection
# invalidates the rest).  Synthetic "models": a first-order Markov chain, so
# the target row (and the draft row) for a context is the table row of its
# last token.

def draft_uniform(seed: int, request_id: int, step: int, position: int) -> float:
    """Uniform for the draft token at `position`: word 2 of the Philox block of
    counter (position, request_id, step, 0), whose words 0 and 1 feed that
    position's accept test and draw (reading: the drafter samples on the
    verifier's stream)."""
    w = philox([position, request_id, step, 0], [seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF])
    return u24(int(w[2]))


def sample_draft(Q_row, T: float, u: float) -> tuple[int, float]:
    """The drafter's token: inverse CDF of softmax(Q / T) at u; arg max at T = 0."""
    if T == 0.0:
        return argmax(Q_row), float("inf")
    return sample_target(Q_row, T, u)


def markov_decode(P_table, Q_table, start, D: int, temperature, steps: int, seed: int = 0,
                  request_id=None):
    """Runs `steps` decode steps for every request: draft D tokens from the
    draft table (row = previous token), verify them against the target table
    rows of the same contexts, keep the emitted tokens, continue from the last
    one.  Returns per-step lists of emitted tokens, accepted lengths, the
    drafts and each request's (draft, accept, draw) margins, the smallest
    margins met, and after each step the running statistics of
    accept_accumulate (the totals and the summary: MAL, expected MAL (0 here:
    no acceptance rates), mean acceptance, P(tau >= k))."""
    P_table = _f32(P_table)
    Q_table = _f32(Q_table)
    B = len(start)
    rid = list(range(B)) if request_id is None else [int(x) for x in request_id]
    last = [int(t) for t in start]
    emitted, taus, drafts, step_margins, step_stats = [], [], [], [], []
    accum = None
    min_margin = {"draft": float("inf"), "accept": float("inf"), "draw": float("inf")}
    for step in range(steps):
        em_s, tau_s, dr_s, mg_s = [], [], [], []
        for r in range(B):
            T = float(temperature[r])
            ctx = [last[r]]
            d = []
            dmin = float("inf")
            for k in range(D):
                y, m = sample_draft(Q_table[ctx[-1]], T, draft_uniform(seed, rid[r], step, k))
                dmin = min(dmin, m)
                d.append(y)
                ctx.append(y)
            min_margin["draft"] = min(min_margin["draft"], dmin)
            ua = [uniforms(seed, rid[r], step, k)[0] for k in range(D)]
            us = [uniforms(seed, rid[r], step, k)[1] for k in range(D + 1)]
            tau, out, am, dm, bits = verify_request(P_table[ctx], Q_table[ctx[:D]] if D else None,
                                                    d, T, ua, us)
            if bits:
                raise ValueError(f"invalid request in the decode loop (bits {bits})")
            min_margin["accept"] = min(min_margin["accept"], am)
            min_margin["draw"] = min(min_margin["draw"], dm)
            em_s.append([int(x) for x in out])
            tau_s.append(int(tau))
            dr_s.append(d)
            mg_s.append((dmin, am, dm))
            last[r] = int(out[-1])
        emitted.append(em_s)
        taus.append(tau_s)
        drafts.append(dr_s)
        step_margins.append(mg_s)
        accum, summ = accept_accumulate(np.full(B, D, np.int32), None, np.asarray(tau_s, np.int32),
                                        D, accum)
        step_stats.append((accum.copy(), summ))
    return dict(emitted=emitted, tau=taus, drafts=drafts, margins=min_margin,
                step_margins=step_margins, step_stats=step_stats)
