"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded synthetic inputs, for the five workloads (c1 tiny, c2 MTP chat,
c3 block at T = 0 and T = 1, c4 budget, c5 mixed temperature) and the full
64 x 16 x 151936 bf16 batch the benchmark times, every request of each
against the oracle (its requests spread over a pool of host threads)."""
import numpy as np
import pytest
import torch

import oracle
from lossless_draft_verification_softmax_amd import specverify as sv
from lossless_draft_verification_softmax_amd import synth
from tests.parity import (compare, gpu_verify, host_f32, oracle_verify_parallel,
                          padded_offsets)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sv.load()


def full_depth_case(name, B=None, V=None, seeds=(0,), sample=None, flags=0):
    w = synth.make(name, device=DEV, B=B, V=V)
    tr0, dr0 = padded_offsets(w.B, w.D, DEV)
    depth = torch.full((w.B,), w.D, dtype=torch.int32, device=DEV)
    th, dh = host_f32(w.target).reshape(-1, w.V), host_f32(w.draft).reshape(-1, w.V)
    temps = w.temperature.cpu().numpy()
    reqs = np.arange(w.B) if sample is None else np.asarray(sample)
    reports = []
    for seed in seeds:
        g = gpu_verify(w.target, w.draft, tr0, dr0, w.draft_tokens, depth, w.temperature,
                       seed=seed, flags=flags)
        o = oracle_verify_parallel(th, dh, tr0.cpu().numpy(), dr0.cpu().numpy(),
                                   w.draft_tokens.cpu().numpy(), depth.cpu().numpy(), temps, reqs,
                                   seed=seed)
        reports.append(compare(g, o, reqs, temps, depth.cpu().numpy()))
    return reports


def test_c1_tiny_t1_many_seeds():
    reps = full_depth_case("c1", seeds=range(40))
    assert sum(r["mismatched"] for r in reps) == 0


def test_c1_tiny_t0():
    full_depth_case("c1_t0", seeds=range(3))


def test_c2_mtp_chat():
    rep = full_depth_case("c2", seeds=(0, 1))
    print(rep)


def test_c2_forced_fp64_draws():
    rep = full_depth_case("c2", seeds=(0,), flags=sv.SV_FLAG_FORCE_FP64_DRAW)
    assert rep[0]["fp64_draws"] == rep[0]["requests"]


def test_c2_forced_fp64_draws_exact_masses():
    """Every float64 tile mass computed directly instead of from the one-pass
    split; the draws must match the oracle the same way."""
    rep = full_depth_case("c2", seeds=(0, 1),
                          flags=sv.SV_FLAG_FORCE_FP64_DRAW | sv.SV_FLAG_EXACT_FP64_MASSES)
    assert all(r["fp64_draws"] == r["requests"] for r in rep)


def test_c4full_forced_fp64_draws_sampled():
    """Float64 draws on full 151936-entry rows (75 tiles), split against direct."""
    a = budget_case("c4full", sample=[0, 17, 45, 63], flags=sv.SV_FLAG_FORCE_FP64_DRAW)[1]
    b = budget_case("c4full", sample=[0, 17, 45, 63],
                    flags=sv.SV_FLAG_FORCE_FP64_DRAW | sv.SV_FLAG_EXACT_FP64_MASSES)[1]
    assert np.array_equal(a["out_tokens"], b["out_tokens"])


def test_c3_block_t0_full():
    full_depth_case("c3_t0")


def test_c3_block_t1_full():
    rep = full_depth_case("c3")
    print(rep)


def test_flag_rate_many_draws():
    """Draws the oracle flags (accept margin under 1e-5, CDF margin under
    1e-12) stay below 1e-4 of all draws over many seeds of the MTP-chat and
    block workloads, and every unflagged draw matches the oracle."""
    reps = full_depth_case("c2", seeds=range(2, 222)) + full_depth_case("c3", seeds=(1, 2, 3, 4))
    draws = sum(r["draws"] for r in reps)
    flagged = sum(r["flagged"] for r in reps)
    literal = sum(r["flagged_literal"] for r in reps)
    print(f"draws={draws} flagged={flagged} flagged_literal_1e-5={literal} "
          f"mismatched={sum(r['mismatched'] for r in reps)} "
          f"fp64_draws={sum(r['fp64_draws'] for r in reps)} "
          f"max_draw_margin_err32={max(r['max_draw_margin_err32'] for r in reps):.3g}")
    assert draws > 10000
    assert flagged < 1e-4 * draws


def budget_case(name, sample=None, packed=True, flags=0):
    w = synth.make(name, device=DEV)
    conf = w.conf.to(DEV).contiguous()
    bud = sv.allocate_budget(conf, w.K)
    torch.cuda.synchronize()
    ob = oracle.allocate_budget(w.conf.numpy(), w.K)
    depth = bud["depth"].cpu().numpy()
    assert np.array_equal(depth, ob["depth"])
    assert np.array_equal(bud["draft_row0"].cpu().numpy(), ob["draft_row0"])
    assert np.array_equal(bud["target_row0"].cpu().numpy(), ob["target_row0"])
    util = bud["utility"].cpu().numpy().astype(np.float64)
    assert np.allclose(util, ob["utility"], rtol=1e-5)
    # Target logits for the kept positions only (packed, as a target forward
    # over the surviving tokens would produce them); draft logits padded.
    B, D, V = w.B, w.D, w.V
    tr0_pad, dr0 = padded_offsets(B, D, DEV)
    if packed:
        idx = torch.cat([torch.arange(int(n) + 1, device=DEV) + r * (D + 1)
                         for r, n in enumerate(depth)])
        target = w.target.reshape(-1, V).index_select(0, idx).contiguous()
        tr0 = bud["target_row0"]
    else:
        target, tr0 = w.target, tr0_pad
    g = gpu_verify(target, w.draft, tr0, dr0, w.draft_tokens, bud["depth"], w.temperature,
                   flags=flags)
    th, dh = host_f32(target).reshape(-1, V), host_f32(w.draft).reshape(-1, V)
    temps = w.temperature.cpu().numpy()
    reqs = np.arange(B) if sample is None else np.asarray(sample)
    o = oracle_verify_parallel(th, dh, tr0.cpu().numpy(), dr0.cpu().numpy(),
                               w.draft_tokens.cpu().numpy(), depth, temps, reqs)
    return compare(g, o, reqs, temps, depth), g, depth


def test_c4_budget_ragged():
    rep, _, depth = budget_case("c4")
    assert depth.sum() == 256
    print(rep)


def test_c4_packed_equals_padded():
    _, g1, _ = budget_case("c4", sample=[0, 40], packed=True)
    _, g2, _ = budget_case("c4", sample=[0, 40], packed=False)
    for k in ("accepted_len", "out_tokens", "num_out", "alpha", "bits"):
        assert np.array_equal(g1[k], g2[k])


def test_c5_mixed_temperature_full():
    rep, _, _ = budget_case("c5")
    print(rep)


def test_c4full_bench_config_full():
    """The batch the benchmark times: 64 x 16 x 151936 bf16 at K = 1024 (every
    position), through the budget and the packed row offsets it returns;
    every request against the oracle."""
    rep, g, depth = budget_case("c4full")
    print(rep)
    assert np.all(depth == 16)
    assert np.all(g["num_out"] == g["accepted_len"] + 1)


@pytest.mark.parametrize("name,sample", [("c2", None), ("c3_t0", None), ("c3", [0, 5, 13])])
def test_streaming_row_pass(name, sample):
    """The streaming row pass (each row pair read twice) instead of the team pass."""
    full_depth_case(name, sample=sample, flags=sv.SV_FLAG_STREAMING_ROW_PASS)


def test_streaming_row_pass_budget_ragged():
    budget_case("c4", flags=sv.SV_FLAG_STREAMING_ROW_PASS)
