"""The team row pass when a team is not all resident at once: a member whose
team wait expires streams the row pair's full rows itself.  The test flag
SV_FLAG_TEAM_WAIT_GIVE_UP makes every wait give up at once (no kernel waits,
faults or hangs: each member simply takes the fallback for every pair), and
the results must still meet the oracle bar, with the timeout reported as
information only."""
import numpy as np
import pytest
import torch

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


def _case(name, B, V, seed):
    w = synth.make(name, device=DEV, B=B, V=V)
    tr0, dr0 = padded_offsets(w.B, w.D, DEV)
    g = torch.Generator().manual_seed(seed)
    depth = torch.randint(0, w.D + 1, (w.B,), generator=g, dtype=torch.int32).to(DEV)
    return w, tr0, dr0, depth


@pytest.mark.parametrize("name,B,V", [("c3", 8, 151936), ("c5", 12, 65536), ("c2", 6, 128000)])
def test_give_up_matches_oracle(name, B, V):
    w, tr0, dr0, depth = _case(name, B, V, seed=B)
    print(f"team fallback: {name} B={B} D={w.D} V={V}", flush=True)
    g = gpu_verify(w.target, w.draft, tr0, dr0, w.draft_tokens, depth, w.temperature, seed=5,
                   flags=sv.SV_FLAG_TEAM_WAIT_GIVE_UP)
    # every request with a drafted position at T > 0 went through a team wait
    waited = (depth.cpu().numpy() > 0) & (w.temperature.cpu().numpy() > 0)
    if waited.any():
        assert np.all(g["bits"] & sv.BIT_SYNC_TIMEOUT)
    th, dh = host_f32(w.target).reshape(-1, V), host_f32(w.draft).reshape(-1, V)
    temps = w.temperature.cpu().numpy()
    reqs = np.arange(w.B)
    o = oracle_verify_parallel(th, dh, tr0.cpu().numpy(), dr0.cpu().numpy(),
                               w.draft_tokens.cpu().numpy(), depth.cpu().numpy(), temps, reqs,
                               seed=5)
    print(compare(g, o, reqs, temps, depth.cpu().numpy()))
    # and the normal team pass gives the same tokens
    n = gpu_verify(w.target, w.draft, tr0, dr0, w.draft_tokens, depth, w.temperature, seed=5)
    assert not np.any(n["bits"] & sv.BIT_SYNC_TIMEOUT)
    assert np.array_equal(n["out_tokens"], g["out_tokens"])
    assert np.allclose(n["alpha"], g["alpha"], rtol=2e-6, atol=1e-7)


def test_give_up_sharded():
    w, tr0, dr0, depth = _case("c3", 6, 151936, seed=3)
    V, W = w.V, 18992
    print(f"team fallback sharded: B={w.B} V={V} shards of {W}", flush=True)

    def split(rows):
        out = []
        for s in range(0, V, W):
            buf = torch.empty((rows.shape[0], W), dtype=rows.dtype, device=rows.device)
            part = rows[:, s:s + W]
            buf[:, : part.shape[1]] = part
            out.append(buf)
        return out

    ts, ds = split(w.target.reshape(-1, V)), split(w.draft.reshape(-1, V))
    outs = []
    for flags in (0, sv.SV_FLAG_TEAM_WAIT_GIVE_UP):
        v = sv.Verifier(w.B, w.D, V, DEV)
        v.prepare_sharded(ts, ds, W, tr0, dr0, w.draft_tokens, depth, w.temperature, seed=2,
                          flags=flags)
        o = v.run()
        torch.cuda.synchronize()
        outs.append((o.out_tokens.cpu().numpy(), o.alpha.cpu().numpy(), o.diag[:, 2].cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.allclose(outs[0][1], outs[1][1], rtol=2e-6, atol=1e-7)
    assert not np.any(outs[0][2] & sv.BIT_SYNC_TIMEOUT)
    if np.any(depth.cpu().numpy() > 0):
        assert np.all(outs[1][2] & sv.BIT_SYNC_TIMEOUT)
