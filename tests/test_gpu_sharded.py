"""Vocabulary-sharded verification (sv_verify_batch_sharded): the rows split
over S separate buffers, as a tensor-parallel target leaves them, give the
verification of the concatenated rows -- against the oracle on the
concatenation (the usual parity bar) and against the unsharded GPU call
(identical tokens and lengths, acceptance rates within float32 rounding).
Covers TP = 8 at V = 151936 bf16, a ragged last shard, fp32, greedy
requests (arg max indices across shards), no draft shards, and the float64
draw path."""
import numpy as np
import pytest
import torch

from lossless_draft_verification_softmax_amd import specverify as sv
from tests.parity import compare, oracle_verify, padded_offsets

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sv.load()


def shard(rows: torch.Tensor, W: int):
    """Separate buffers of W columns (the last one narrower), stride W."""
    out = []
    for s in range(0, rows.shape[1], W):
        buf = torch.full((rows.shape[0], W), float("nan"), dtype=rows.dtype, device=rows.device)
        part = rows[:, s:s + W]
        buf[:, : part.shape[1]] = part
        out.append(buf)
    return out


def outputs(out):
    torch.cuda.synchronize()
    am, dm = out.margins()
    return dict(accepted_len=out.accepted_len.cpu().numpy(),
                out_tokens=out.out_tokens.cpu().numpy(), num_out=out.num_out.cpu().numpy(),
                alpha=None if out.alpha is None else out.alpha.cpu().numpy().copy(),
                bits=out.bits().cpu().numpy().astype(np.uint32),
                accept_margin=am.cpu().numpy(), draw_margin=dm.cpu().numpy())


def batch(rng, B, D, V, dtype, temps, noise=1.0):
    P = (3.0 * rng.standard_normal((B * (D + 1), V))).astype(np.float32)
    Q = np.empty((B * D, V), np.float32)
    for r in range(B):
        for k in range(D):
            Q[r * D + k] = P[r * (D + 1) + k] + noise * rng.standard_normal(V)
    Pt = torch.from_numpy(P).to(dtype).to(DEV)
    Qt = torch.from_numpy(Q).to(dtype).to(DEV)
    tok = torch.from_numpy(rng.integers(0, V, size=(B, D)).astype(np.int32)).to(DEV)
    depth = torch.from_numpy(rng.integers(0, D + 1, size=B).astype(np.int32)).to(DEV)
    T = torch.from_numpy(np.asarray(temps, np.float32)).to(DEV)
    return Pt, Qt, tok, depth, T


def run_case(rng, B, D, V, W, dtype, temps, flags=0, with_draft=True):
    Pt, Qt, tok, depth, T = batch(rng, B, D, V, dtype, temps)
    tr0, dr0 = padded_offsets(B, D, DEV)
    ref = sv.Verifier(B, D, V, DEV).prepare(Pt, Qt if with_draft else None, tr0,
                                            dr0 if with_draft else None, tok, depth, T, seed=3,
                                            flags=flags)
    want = outputs(ref.run())
    ts = shard(Pt, W)
    ds = shard(Qt, W) if with_draft else None
    v = sv.Verifier(B, D, V, DEV).prepare_sharded(ts, ds, W, tr0, dr0 if with_draft else None,
                                                  tok, depth, T, seed=3, flags=flags)
    got = outputs(v.run())
    # the same tokens and lengths as the unsharded call
    assert np.array_equal(got["accepted_len"], want["accepted_len"])
    assert np.array_equal(got["out_tokens"], want["out_tokens"])
    assert np.array_equal(got["bits"] & ~np.uint32(sv.BIT_FP64_DRAW),
                          want["bits"] & ~np.uint32(sv.BIT_FP64_DRAW))
    if with_draft:
        assert np.allclose(got["alpha"], want["alpha"], rtol=2e-6, atol=1e-7)
    # and parity with the oracle on the concatenated rows
    Ph = Pt.float().cpu().numpy()
    Qh = Qt.float().cpu().numpy() if with_draft else None
    reqs = np.arange(B)
    orc = oracle_verify(Ph, Qh, tr0.cpu().numpy(), dr0.cpu().numpy() if with_draft else None,
                        tok.cpu().numpy(), depth.cpu().numpy(), T.cpu().numpy(), reqs, seed=3)
    rep = compare(got, orc, reqs, T.cpu().numpy(), depth.cpu().numpy(), check_alpha=with_draft)
    return rep


def test_tp8_bf16_full_vocab():
    rng = np.random.default_rng(41)
    rep = run_case(rng, 8, 4, 151936, 18992, torch.bfloat16, [1.0] * 6 + [0.0, 0.7])
    assert rep["mismatched"] == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_last_shard_mixed_temperatures(dtype):
    rng = np.random.default_rng(42)
    run_case(rng, 10, 3, 40000, 8192, dtype, [1.0, 0.0, 0.6, 1.3, 0.0, 1.0, 2.0, 0.9, 1.0, 0.0])


def test_greedy_without_draft_shards():
    rng = np.random.default_rng(43)
    run_case(rng, 6, 3, 30000, 4096, torch.bfloat16, [0.0] * 6, with_draft=False)


def test_forced_float64_draws_and_one_shard():
    rng = np.random.default_rng(44)
    run_case(rng, 6, 2, 50000, 12504, torch.bfloat16, [1.0] * 6, flags=sv.SV_FLAG_FORCE_FP64_DRAW)
    run_case(rng, 4, 2, 5000, 5000, torch.float32, [1.0] * 4)
