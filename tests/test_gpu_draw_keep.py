"""Float64 draws whose tiles hold elements of uncertain residual sign.

The one-pass split of the float64 tile pass sorts each element of a residual
draw row by d = ep rho_e - eq: certainly positive, certainly not, equal
logits, or within the band |d| <= 1e-4 ep rho_e.  An element in the band
keeps its (ep, eq) for the pick, up to 16 per tile; the pick reads the first
four together with its first loads, the rest afterwards, and recomputes a
tile with more than 16 directly.  Synthetic rows rarely put anything in the
band, so these fp32 rows are built to:
- the draft row equals the target row except in four places;
- a block A lowered by 1 carries the residual mass;
- the drafted token, raised by 6, is almost always rejected, so the draw
  is a residual draw at position 0;
- in every tile, k elements are raised by a few float32 ulps (p and q
  within about 1e-6 of each other: in the band once the two normalisers
  agree);
- a block B is shifted so that sum exp(draft) equals sum exp(target).
  Then Zq / Zp equals kappa, the ratio that equal logits have, and the
  raised elements fall in the band.

k is 3, 9 or 20 by request, so every path of the pick's kept elements runs.
Every draw is forced into float64; the tokens must match the oracle's as in
the other parity tests, and the tile masses taken directly
(SV_FLAG_EXACT_FP64_MASSES) must give the same tokens.
"""
import numpy as np
import pytest
import torch

from lossless_draft_verification_softmax_amd import specverify as sv
from tests.parity import compare, gpu_verify, oracle_verify_parallel, padded_offsets

pytestmark = pytest.mark.gpu

DEV = "cuda"
TILE = 2048
KEEP_PER_TILE = (3, 9, 20)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sv.load()


def keep_rows(B, V, seed):
    """Target rows [B, 2, V] (position 0, bonus), draft rows [B, 1, V], drafted
    tokens [B, 1], all fp32."""
    rng = np.random.default_rng(seed)
    target = rng.standard_normal((B, 2, V)).astype(np.float32)
    draft = target[:, :1, :].copy()
    tokens = np.zeros((B, 1), dtype=np.int32)
    ntiles = (V + TILE - 1) // TILE
    for r in range(B):
        x = target[r, 0].astype(np.float64)
        y = draft[r, 0]
        a0 = int(rng.integers(0, V - 600))
        A = np.arange(a0, a0 + 512)
        y[A] = (x[A] - 1.0).astype(np.float32)
        taken = np.zeros(V, dtype=bool)
        taken[A] = True
        # a drafted token with x < -0.5: raising it adds little mass
        d0 = int(rng.choice(np.flatnonzero(~taken & (x < -0.5))))
        tokens[r, 0] = d0
        y[d0] = np.float32(x[d0] + 6.0)
        taken[d0] = True
        k = KEEP_PER_TILE[r % len(KEEP_PER_TILE)]
        for t in range(ntiles):
            lo, hi = t * TILE, min(V, (t + 1) * TILE)
            free = np.flatnonzero(~taken[lo:hi]) + lo
            pick = rng.choice(free, size=min(k, free.size), replace=False)
            for i in pick:
                v = np.float32(x[i])
                for _ in range(int(rng.integers(2, 6))):
                    v = np.nextafter(v, np.float32(np.inf) if rng.random() < 0.5 else np.float32(-np.inf))
                y[i] = v
            taken[pick] = True
        # block B restores sum exp(draft) = sum exp(target), in float64
        free = np.flatnonzero(~taken)
        b0 = int(rng.integers(0, free.size - 2048))
        Bi = free[b0:b0 + 2048]
        yd = y.astype(np.float64)
        need = np.exp(x).sum() - (np.exp(yd).sum() - np.exp(yd[Bi]).sum())
        c = np.log(need / np.exp(x[Bi]).sum())
        y[Bi] = (x[Bi] + c).astype(np.float32)
    return target, draft, tokens


@pytest.mark.parametrize("V", [20000, 2 * TILE * 5])
def test_forced_fp64_draws_with_kept_elements(V):
    B, D = 24, 1
    for seed in (0, 1):
        target, draft, tokens = keep_rows(B, V, seed)
        tgt = torch.from_numpy(target.reshape(B * (D + 1), V)).to(DEV)
        dft = torch.from_numpy(draft.reshape(B * D, V)).to(DEV)
        tok = torch.from_numpy(tokens).to(DEV)
        tr0, dr0 = padded_offsets(B, D, DEV)
        depth = torch.full((B,), D, dtype=torch.int32, device=DEV)
        temps = torch.ones(B, dtype=torch.float32, device=DEV)
        flags = sv.SV_FLAG_FORCE_FP64_DRAW
        g = gpu_verify(tgt, dft, tr0, dr0, tok, depth, temps, seed=seed, flags=flags)
        gx = gpu_verify(tgt, dft, tr0, dr0, tok, depth, temps, seed=seed,
                        flags=flags | sv.SV_FLAG_EXACT_FP64_MASSES)
        reqs = np.arange(B)
        o = oracle_verify_parallel(target.reshape(B * (D + 1), V), draft.reshape(B * D, V),
                                   tr0.cpu().numpy(), dr0.cpu().numpy(), tokens,
                                   depth.cpu().numpy(), temps.cpu().numpy(), reqs, seed=seed)
        rep = compare(g, o, reqs, temps.cpu().numpy(), depth.cpu().numpy(), check_flag_rate=False)
        assert rep["fp64_draws"] == B, rep
        # the drafted token is rejected almost surely: residual draws
        assert (g["accepted_len"] == 0).sum() >= B - 2, g["accepted_len"]
        assert np.array_equal(g["out_tokens"], gx["out_tokens"]), (g["out_tokens"], gx["out_tokens"])
        print(f"V={V} seed={seed}: {rep}")
