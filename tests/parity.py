"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI,
run the CPU oracle on the same inputs (copied to the host), and compare.

Acceptance bar (element by element):
  * T = 0 requests, budget depths / row offsets, invalid-request handling:
    bit-exact.
  * T > 0: accepted length and emitted tokens bit-exact, except for requests
    the oracle flags: an accept test with |u - p/q| < 1e-5, or a draw whose
    long-double CDF boundary distance is below 1e-12 (the GPU recomputes
    every draw within 1e-5 of a boundary in float64, so only draws within
    float64 rounding of a boundary may differ).  The count of draws inside
    the literal 1e-5 CDF band is reported as well.
  * alpha within 1e-5 relative (plus 1e-7 absolute for alpha near 0).
  * The draws the oracle flags are fewer than 1e-4 of all draws (uniforms
    consumed) of the compared requests, on the workloads (constructed edge
    rows, which put draws on boundaries on purpose, skip this count).
  * The GPU's accept margin min_k |u_k - p_k(d)/q_k(d)| agrees with the
    oracle's to within 1e-5 of the ratio (the accept ratio within 1e-5
    relative); its draw margin (distance of u R to the nearest CDF boundary)
    to within the float32 draw's error budget, or float64 rounding for a draw
    recomputed in float64.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from lossless_draft_verification_softmax_amd import specverify as sv

ACCEPT_BAND = 1e-5
DRAW_BAND = 1e-12
DRAW_BAND_LITERAL = 1e-5
ALPHA_RTOL = 1e-5
ALPHA_ATOL = 1e-7
FLAG_RATE = 1e-4
# Accept ratio within 1e-5 relative: |margin_gpu - margin_oracle| <= 1e-5 ratio
# <= 1e-5 (margin + 1), since ratio <= margin + u and u < 1.
ACCEPT_MARGIN_RTOL = 1e-5
# Draw margins, absolute in probability units: the float32 draw's error
# budget (normaliser, exponent-argument and exp2 rounding, tile scans), and
# float64 rounding for draws the GPU recomputed in float64 (the margin is
# stored as a float32, so 1e-7 relative).
DRAW_MARGIN_ATOL32 = 5e-6
DRAW_MARGIN_RTOL64 = 1e-7
DRAW_MARGIN_ATOL64 = 1e-12


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def gpu_verify(target, draft, target_row0, draft_row0, tokens, depth, temperature, *, seed=0,
               step=0, request_id=None, flags=0, V=None):
    out = sv.verify(target, draft, target_row0, draft_row0, tokens, depth, temperature, seed=seed,
                    step=step, request_id=request_id, flags=flags, V=V)
    torch.cuda.synchronize()
    am, dm = out.margins()
    return dict(accepted_len=out.accepted_len.cpu().numpy(),
                out_tokens=out.out_tokens.cpu().numpy(),
                num_out=out.num_out.cpu().numpy(),
                alpha=None if out.alpha is None else out.alpha.cpu().numpy(),
                bits=out.bits().cpu().numpy().astype(np.uint32),
                accept_margin=am.cpu().numpy(), draw_margin=dm.cpu().numpy())


def oracle_verify(target_h, draft_h, target_row0, draft_row0, tokens, depth, temperature,
                  requests, *, seed=0, step=0, request_id=None, D_max=None):
    """Oracle on a subset of requests, keeping each request's own Philox
    stream (request_id = original index unless given)."""
    requests = np.asarray(requests, dtype=np.int64)
    tr0 = np.asarray(target_row0)[requests]
    dr0 = np.asarray(draft_row0)[requests] if draft_row0 is not None else None
    tok = np.ascontiguousarray(np.asarray(tokens)[requests])
    dep = np.asarray(depth)[requests]
    temp = np.asarray(temperature)[requests]
    rid = (np.asarray(request_id)[requests] if request_id is not None else requests).astype(np.uint32)
    return oracle.verify_batch(target_h, draft_h, tr0, dr0, tok, dep, temp, seed=seed, step=step,
                               request_id=rid, D_max=D_max if D_max is not None else tok.shape[1])


def oracle_verify_parallel(target_h, draft_h, target_row0, draft_row0, tokens, depth,
                           temperature, requests, *, workers=None, **kw):
    """oracle_verify over every given request, one request per call on a pool
    of host threads (the oracle's C calls run outside the GIL), the results
    concatenated in request order."""
    import concurrent.futures
    import os
    requests = [int(r) for r in requests]
    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(lambda r: oracle_verify(target_h, draft_h, target_row0, draft_row0,
                                                    tokens, depth, temperature, [r], **kw),
                            requests))
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


def compare(gpu: dict, orc: dict, requests, temperature, depth, *, check_alpha=True,
            check_flag_rate=True, check_margins=True) -> dict:
    """Assert parity on the given requests; return counts for reporting."""
    requests = np.asarray(requests)
    temperature = np.asarray(temperature)
    depth = np.asarray(depth)
    rep = dict(requests=len(requests), draws=0, accept_draws=0, flagged=0, flagged_literal=0,
               mismatched=0, fp64_draws=0, max_accept_margin_err=0.0, max_draw_margin_err32=0.0,
               max_draw_margin_err64=0.0)
    for i, r in enumerate(requests):
        T = float(temperature[r])
        bits_o = int(orc["bits"][i])
        # informational bits: the float64 draw, a zero residual (the oracle
        # reports it too), a team wait that fell back to the full rows
        bits_g = int(gpu["bits"][r]) & ~(sv.BIT_FP64_DRAW | sv.BIT_RESIDUAL_ZERO |
                                         sv.BIT_SYNC_TIMEOUT)
        assert bits_g == (bits_o & ~oracle.BIT_RESIDUAL_ZERO), (r, bits_g, bits_o)
        same = (gpu["accepted_len"][r] == orc["accepted_len"][i]
                and gpu["num_out"][r] == orc["num_out"][i]
                and np.array_equal(gpu["out_tokens"][r], orc["out_tokens"][i]))
        if int(gpu["bits"][r]) & sv.BIT_FP64_DRAW:
            rep["fp64_draws"] += 1
        if T == 0.0 or bits_o:
            assert same, (r, T, gpu["out_tokens"][r], orc["out_tokens"][i])
        else:
            rep["draws"] += int(orc["draws"][i])
            rep["accept_draws"] += int(orc["draws"][i]) - 1
            flagged = (orc["accept_margin"][i] < ACCEPT_BAND or orc["draw_margin"][i] < DRAW_BAND)
            literal = (orc["accept_margin"][i] < ACCEPT_BAND
                       or orc["draw_margin"][i] < DRAW_BAND_LITERAL)
            rep["flagged"] += int(flagged)
            rep["flagged_literal"] += int(literal)
            if not same:
                rep["mismatched"] += 1
                assert flagged, (r, gpu["out_tokens"][r], orc["out_tokens"][i],
                                 orc["accept_margin"][i], orc["draw_margin"][i])
            elif check_margins and "accept_margin" in gpu:
                _check_margins(gpu, orc, r, i, rep)
        if check_alpha and gpu["alpha"] is not None and not bits_o:
            n = int(depth[r])
            ga = gpu["alpha"][r, :n].astype(np.float64)
            oa = orc["alpha"][i, :n]
            assert np.all(np.abs(ga - oa) <= ALPHA_RTOL * np.abs(oa) + ALPHA_ATOL), (r, ga, oa)
            assert np.all(gpu["alpha"][r, n:] == 0.0)
    if check_flag_rate:
        assert rep["flagged"] < FLAG_RATE * max(rep["draws"], 1) or rep["flagged"] == 0, rep
    return rep


def _check_margins(gpu, orc, r, i, rep):
    """Margins of a request whose outputs agree with the oracle's.  A margin
    the oracle puts inside its flag band is not compared: there the decision
    itself may go either way (and a float64 residual that vanishes takes the
    draw from p), so the two margins need not be close."""
    ga, oa = float(gpu["accept_margin"][r]), float(orc["accept_margin"][i])
    if oa < ACCEPT_BAND:
        pass
    elif np.isinf(oa) or np.isinf(ga):
        assert np.isinf(oa) and np.isinf(ga), (r, ga, oa)
    else:
        err = abs(ga - oa)
        rep["max_accept_margin_err"] = max(rep["max_accept_margin_err"], err)
        assert err <= ACCEPT_MARGIN_RTOL * (oa + 1.0), (r, ga, oa)
    gd, od = float(gpu["draw_margin"][r]), float(orc["draw_margin"][i])
    err = abs(gd - od)
    if od < DRAW_BAND:
        return
    if int(gpu["bits"][r]) & sv.BIT_FP64_DRAW:
        rep["max_draw_margin_err64"] = max(rep["max_draw_margin_err64"], err)
        assert err <= DRAW_MARGIN_RTOL64 * od + DRAW_MARGIN_ATOL64, (r, gd, od)
    else:
        rep["max_draw_margin_err32"] = max(rep["max_draw_margin_err32"], err)
        assert err <= DRAW_MARGIN_ATOL32, (r, gd, od)


def padded_offsets(B: int, D: int, device):
    tr0 = torch.arange(B, dtype=torch.int64, device=device) * (D + 1)
    dr0 = torch.arange(B, dtype=torch.int64, device=device) * D
    return tr0, dr0
