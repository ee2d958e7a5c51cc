"""GPU property and edge-case tests against the oracle: random shapes with
padded row strides (NaN in the padding, which must never be read), ragged
and zero depths, mixed temperatures, both dtypes, invalid inputs, request
ids / seeds / steps, the budget on adversarial confidences, the statistics,
and run-to-run determinism."""
import numpy as np
import pytest
import torch

import oracle
from lossless_draft_verification_softmax_amd import specverify as sv
from lossless_draft_verification_softmax_amd import synth
from tests.parity import compare, gpu_verify, oracle_verify, padded_offsets

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sv.load()


def random_batch(rng, B, D, V, stride, dtype, temps, scale=2.5, noise=1.0, mask_frac=0.0):
    rows_t, rows_d = B * (D + 1), max(B * D, 1)
    P = (scale * rng.standard_normal((rows_t, stride))).astype(np.float32)
    Q = np.empty((rows_d, stride), np.float32)
    for r in range(B):
        for k in range(D):
            Q[r * D + k] = P[r * (D + 1) + k] + noise * rng.standard_normal(stride)
    if mask_frac > 0:
        P[rng.random(P.shape) < mask_frac] = -np.inf
        Q[rng.random(Q.shape) < mask_frac] = -np.inf
        P[:, 0] = 0.0  # keep every row valid
        Q[:, 0] = 0.0
    P[:, V:] = np.nan  # padding: never read
    Q[:, V:] = np.nan
    tokens = rng.integers(0, V, size=(B, max(D, 1))).astype(np.int32)[:, :D].copy()
    for r in range(B):  # greedy drafts for T = 0 requests, often matching
        if temps[r] == 0.0:
            for k in range(D):
                row = P[r * (D + 1) + k, :V]
                if rng.random() < 0.8:
                    tokens[r, k] = int(np.argmax(row.astype(dtype_np(dtype))))
    return P, Q, tokens


def dtype_np(dtype):
    return np.float32


def to_dev(P, dtype):
    return torch.from_numpy(P).to(DEV).to(dtype)


@pytest.mark.parametrize("row_pass", ["team", "stream"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("trial", range(8))
def test_random_shapes(dtype, trial, row_pass):
    rng = np.random.default_rng(100 + trial)
    B = int(rng.integers(1, 9))
    D = int(rng.integers(0, 9))
    V = int(rng.choice([1, 7, 33, 1001, 4099, 20000, 70001]))
    vec = 8 if dtype == torch.bfloat16 else 4
    stride = (V + vec - 1) // vec * vec + vec * int(rng.integers(0, 3))
    temps = rng.choice(np.array([0.0, 0.6, 1.0, 1.7], np.float32), size=B)
    P, Q, tokens = random_batch(rng, B, D, V, stride, dtype, temps,
                                mask_frac=0.1 if trial % 3 == 0 else 0.0)
    Pd, Qd = to_dev(P, dtype), to_dev(Q, dtype)
    depth = rng.integers(0, D + 1, size=B).astype(np.int32)
    tr0, dr0 = padded_offsets(B, D, DEV)
    seed, step = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**32))
    rid = rng.integers(0, 2**32, size=B, dtype=np.uint64).astype(np.uint32)
    g = gpu_verify(Pd, Qd, tr0, dr0, torch.from_numpy(tokens).to(DEV).reshape(B, D),
                   torch.from_numpy(depth).to(DEV), torch.from_numpy(temps).to(DEV), seed=seed,
                   step=step, request_id=torch.from_numpy(rid).to(DEV), V=V,
                   flags=sv.SV_FLAG_STREAMING_ROW_PASS if row_pass == "stream" else 0)
    # the oracle sees exactly the device values, rows cut to V
    Ph = Pd.float().cpu().numpy()[:, :V].copy()
    Qh = Qd.float().cpu().numpy()[:, :V].copy()
    o = oracle_verify(Ph, Qh, tr0.cpu().numpy(), dr0.cpu().numpy(), tokens.reshape(B, D), depth,
                      temps, np.arange(B), seed=seed, step=step, request_id=rid, D_max=D)
    rep = compare(g, o, np.arange(B), temps, depth, check_flag_rate=False)
    assert rep["mismatched"] == 0 or rep["flagged"] >= rep["mismatched"]


def test_invalid_inputs():
    rng = np.random.default_rng(7)
    B, D, V = 8, 3, 100
    temps = np.ones(B, np.float32)
    P, Q, tokens = random_batch(rng, B, D, V, V, torch.float32, temps)
    P[1 * (D + 1) + 2, 5] = np.nan          # r1: NaN in a target row
    P[2 * (D + 1) + 3, 7] = np.inf          # r2: +inf in the bonus row
    Q[3 * D + 1, :] = -np.inf               # r3: all -inf draft row
    tokens[4, 2] = V                        # r4: token out of range
    tokens[5, 0] = -3                       # r5: negative token
    depth = np.full(B, D, np.int32)
    depth[6] = D + 1                        # r6: depth beyond D_max
    temps[7] = -1.0                         # r7: negative temperature
    tr0, dr0 = padded_offsets(B, D, DEV)
    g = gpu_verify(to_dev(P, torch.float32), to_dev(Q, torch.float32), tr0, dr0,
                   torch.from_numpy(tokens).to(DEV), torch.from_numpy(depth).to(DEV),
                   torch.from_numpy(temps).to(DEV))
    o = oracle_verify(P, Q, tr0.cpu().numpy(), dr0.cpu().numpy(), tokens, depth, temps,
                      np.arange(B), D_max=D)
    compare(g, o, np.arange(B), temps, depth, check_flag_rate=False)
    assert list(g["bits"][1:8]) == [sv.BIT_BAD_ROW, sv.BIT_BAD_ROW, sv.BIT_BAD_ROW,
                                    sv.BIT_BAD_TOKEN, sv.BIT_BAD_TOKEN, sv.BIT_BAD_DEPTH,
                                    sv.BIT_BAD_TEMPERATURE]
    assert np.all(g["num_out"][1:] == 0) and np.all(g["out_tokens"][1:] == -1)
    assert g["num_out"][0] >= 1


def test_nan_temperature_and_inf_temperature():
    B, D, V = 2, 1, 16
    P = np.zeros((B * (D + 1), V), np.float32)
    Q = np.zeros((B * D, V), np.float32)
    temps = np.array([np.nan, np.inf], np.float32)
    tr0, dr0 = padded_offsets(B, D, DEV)
    g = gpu_verify(to_dev(P, torch.float32), to_dev(Q, torch.float32), tr0, dr0,
                   torch.zeros((B, D), dtype=torch.int32, device=DEV),
                   torch.ones(B, dtype=torch.int32, device=DEV), torch.from_numpy(temps).to(DEV))
    assert np.all(g["bits"] == sv.BIT_BAD_TEMPERATURE)


@pytest.mark.parametrize("row_pass", ["team", "stream"])
def test_temperature_domain_scaled_maximum(row_pass):
    """Requests whose scaled row maximum |m * fl(log2(e)/T)| reaches 2^24
    are invalid on both sides (the domain of the float32 row states); just
    inside it the peaked rows verify bit for bit against the oracle, with
    full-vocabulary rows and the team or streaming pass."""
    rng = np.random.default_rng(44)
    B, D, V = 6, 3, 151936
    P = (3.0 * rng.standard_normal((B * (D + 1), V))).astype(np.float32)
    Q = (P[np.arange(B * (D + 1)).reshape(B, D + 1)[:, :D].reshape(-1)]
         + 0.5 * rng.standard_normal((B * D, V))).astype(np.float32)
    peak = rng.integers(0, V, size=B)
    for r in range(B):
        P[r * (D + 1):(r + 1) * (D + 1), peak[r]] = 100.0
        Q[r * D:(r + 1) * D, peak[r]] = 100.0
    P[1 * (D + 1) + 3, 17] = 120.0      # r1: bonus row past 2^24 at T = 1e-5
    Q[3 * D + 2, :] = -120.0            # r3: an all -120 draft row past it
    temps = np.array([1e-5, 1e-5, 1e-5, 1e-5, 1e-37, 1e-37], np.float32)
    P[5 * (D + 1):6 * (D + 1)] *= 1e-32   # r5: tiny logits stay inside at 1e-37
    Q[5 * D:6 * D] *= 1e-32
    tokens = np.repeat(peak[:, None], D, axis=1).astype(np.int32)
    depth = np.full(B, D, np.int32)
    tr0, dr0 = padded_offsets(B, D, DEV)
    g = gpu_verify(to_dev(P, torch.float32), to_dev(Q, torch.float32), tr0, dr0,
                   torch.from_numpy(tokens).to(DEV), torch.from_numpy(depth).to(DEV),
                   torch.from_numpy(temps).to(DEV),
                   flags=sv.SV_FLAG_STREAMING_ROW_PASS if row_pass == "stream" else 0)
    o = oracle_verify(P, Q, tr0.cpu().numpy(), dr0.cpu().numpy(), tokens, depth, temps,
                      np.arange(B), D_max=D)
    compare(g, o, np.arange(B), temps, depth, check_flag_rate=False)
    assert [int(b) & sv.BIT_BAD_TEMPERATURE for b in g["bits"]] == [
        0, sv.BIT_BAD_TEMPERATURE, 0, sv.BIT_BAD_TEMPERATURE, sv.BIT_BAD_TEMPERATURE, 0]
    for r in (0, 2, 5):
        assert g["accepted_len"][r] == D


def test_degenerate_shapes():
    # empty batch
    out = sv.verify(torch.zeros((1, 8), device=DEV), None, torch.zeros(0, dtype=torch.int64, device=DEV),
                    None, torch.zeros((0, 2), dtype=torch.int32, device=DEV),
                    torch.zeros(0, dtype=torch.int32, device=DEV),
                    torch.zeros(0, dtype=torch.float32, device=DEV))
    assert out.accepted_len.numel() == 0
    # D_max = 0: every request emits exactly its bonus token
    rng = np.random.default_rng(3)
    B, V = 5, 300
    P = rng.standard_normal((B, V)).astype(np.float32)
    temps = np.array([0.0, 1.0, 0.6, 1.0, 0.0], np.float32)
    tr0 = torch.arange(B, dtype=torch.int64, device=DEV)
    g = gpu_verify(to_dev(P, torch.float32), None, tr0, None,
                   torch.zeros((B, 0), dtype=torch.int32, device=DEV),
                   torch.zeros(B, dtype=torch.int32, device=DEV), torch.from_numpy(temps).to(DEV))
    o = oracle_verify(P, None, tr0.cpu().numpy(), None, np.zeros((B, 0), np.int32),
                      np.zeros(B, np.int32), temps, np.arange(B), D_max=0)
    compare(g, o, np.arange(B), temps, np.zeros(B, np.int32), check_flag_rate=False)
    assert np.all(g["num_out"] == 1)
    # V = 1: p = q = 1, every draft kept, bonus token 0
    B, D = 3, 4
    P1 = torch.zeros((B * (D + 1), 8), device=DEV)
    Q1 = torch.zeros((B * D, 8), device=DEV)
    tr0, dr0 = padded_offsets(B, D, DEV)
    g = gpu_verify(P1, Q1, tr0, dr0, torch.zeros((B, D), dtype=torch.int32, device=DEV),
                   torch.full((B,), D, dtype=torch.int32, device=DEV),
                   torch.tensor([1.0, 0.0, 0.5], device=DEV), V=1)
    assert np.all(g["accepted_len"] == D) and np.all(g["out_tokens"] == 0)


def test_draft_logits_absent_with_sampling_request():
    B, D, V = 3, 2, 64
    P = torch.randn((B * (D + 1), V), device=DEV)
    tr0, _ = padded_offsets(B, D, DEV)
    tokens = np.zeros((B, D), np.int32)
    depth = np.array([D, D, 0], np.int32)
    temps = np.array([0.0, 1.0, 1.0], np.float32)
    g = gpu_verify(P, None, tr0, None, torch.from_numpy(tokens).to(DEV),
                   torch.from_numpy(depth).to(DEV), torch.from_numpy(temps).to(DEV))
    assert g["bits"][0] == 0 and g["bits"][1] == sv.BIT_BAD_ROW and g["bits"][2] == 0
    o = oracle_verify(P.cpu().numpy(), None, tr0.cpu().numpy(), None, tokens, depth, temps,
                      np.arange(B))
    compare(g, o, np.arange(B), temps, depth, check_alpha=False, check_flag_rate=False)


def test_identical_draft_accepts_all_on_gpu():
    w = synth.make("c2", device=DEV)
    tr0, dr0 = padded_offsets(w.B, w.D, DEV)
    draft = w.target[:, : w.D].contiguous()
    g = gpu_verify(w.target, draft, tr0, dr0, w.draft_tokens,
                   torch.full((w.B,), w.D, dtype=torch.int32, device=DEV), w.temperature)
    assert np.all(g["accepted_len"] == w.D)
    assert np.allclose(g["alpha"], 1.0, atol=1e-5)


def test_determinism():
    w = synth.make("c2", device=DEV)
    tr0, dr0 = padded_offsets(w.B, w.D, DEV)
    depth = torch.full((w.B,), w.D, dtype=torch.int32, device=DEV)
    outs = [gpu_verify(w.target, w.draft, tr0, dr0, w.draft_tokens, depth, w.temperature, seed=5)
            for _ in range(3)]
    for o in outs[1:]:
        for k in outs[0]:
            assert np.array_equal(outs[0][k], o[k], equal_nan=True), k


@pytest.mark.parametrize("trial", range(12))
def test_budget_random(trial):
    rng = np.random.default_rng(500 + trial)
    B = int(rng.integers(1, 80))
    D = int(rng.integers(1, 65))
    while B * D > 4096:
        D //= 2
    conf = rng.beta(2.0, 1.0, size=(B, D)).astype(np.float32)
    special = rng.random((B, D))
    conf[special < 0.05] = 1.0
    conf[(special >= 0.05) & (special < 0.08)] = 0.0
    conf[(special >= 0.08) & (special < 0.09)] = np.nan
    conf[(special >= 0.09) & (special < 0.10)] = 1.5
    conf[(special >= 0.10) & (special < 0.12)] = 1e-20  # products reach subnormals and zero
    if trial % 3 == 0:
        conf[:] = conf[0]
    K = int(rng.integers(-2, B * D + 5))
    md = rng.integers(-1, D + 2, size=B).astype(np.int32) if trial % 2 else None
    g = sv.allocate_budget(torch.from_numpy(conf).to(DEV), K,
                           None if md is None else torch.from_numpy(md))
    torch.cuda.synchronize()
    o = oracle.allocate_budget(conf, K, md)
    assert np.array_equal(g["depth"].cpu().numpy(), o["depth"])
    assert np.array_equal(g["draft_row0"].cpu().numpy(), o["draft_row0"])
    assert np.array_equal(g["target_row0"].cpu().numpy(), o["target_row0"])
    u = g["utility"].cpu().numpy().astype(np.float64)
    assert np.allclose(u, o["utility"], rtol=1e-5, atol=1e-30)


def test_budget_full_size_configs():
    for name in ("c4", "c5", "c4full"):
        w = synth.make(name, device="cpu", B=None, V=8)
        g = sv.allocate_budget(w.conf.to(DEV), w.K)
        torch.cuda.synchronize()
        o = oracle.allocate_budget(w.conf.numpy(), w.K)
        assert np.array_equal(g["depth"].cpu().numpy(), o["depth"])
        assert np.array_equal(g["target_row0"].cpu().numpy(), o["target_row0"])


def test_accept_stats_match_oracle():
    rng = np.random.default_rng(9)
    for B, D in ((1, 1), (16, 3), (64, 16), (300, 64)):
        depth = rng.integers(0, D + 1, size=B).astype(np.int32)
        tau = np.array([rng.integers(0, n + 1) for n in depth], np.int32)
        alpha = rng.uniform(0, 1, size=(B, D)).astype(np.float32)
        g = sv.accept_stats(torch.from_numpy(depth).to(DEV), torch.from_numpy(alpha).to(DEV),
                            torch.from_numpy(tau).to(DEV), D)
        torch.cuda.synchronize()
        o = oracle.accept_stats(depth, alpha.astype(np.float64), tau, D)
        assert np.allclose(g["expected_len"].cpu().numpy(), o["expected_len"], rtol=1e-5, atol=1e-6)
        assert np.allclose(g["per_depth"].cpu().numpy().reshape(3, D), o["per_depth"], rtol=1e-5,
                           atol=1e-6)
        assert np.allclose(g["summary"].cpu().numpy(), o["summary"], rtol=1e-5)


STATS_CASES = {  # B, D, V, dtype, options
    "tiny": (1, 1, 7, torch.float32, {}),
    "ragged": (37, 5, 1001, torch.bfloat16, {}),
    "wide": (300, 3, 512, torch.float32, {}),
    "depth0": (5, 0, 64, torch.bfloat16, {}),
    "deep": (20, 64, 200, torch.float32, {}),
    "no_alpha": (37, 5, 1001, torch.bfloat16, {"alpha": False}),
    "invalid": (24, 6, 333, torch.float32, {"invalid": True}),
    "stream": (37, 5, 1001, torch.bfloat16, {"flags": sv.SV_FLAG_STREAMING_ROW_PASS}),
    "noalloc": (37, 5, 1001, torch.bfloat16, {"noalloc": True}),
    "sharded": (19, 4, 3000, torch.bfloat16, {"shard": 1024}),
}


def _stats_inputs(case):
    B, D, V, dtype, opt = STATS_CASES[case]
    rng = np.random.default_rng(sum(map(ord, case)))
    vec = 8 if dtype == torch.bfloat16 else 4
    stride = (V + vec - 1) // vec * vec + vec
    temps = rng.choice(np.array([0.0, 0.6, 1.0], np.float32), size=B)
    P, Q, tokens = random_batch(rng, B, D, V, stride, dtype, temps)
    depth = rng.integers(0, D + 1, size=B).astype(np.int32)
    if opt.get("invalid"):
        temps[1] = np.nan     # invalid temperature
        depth[2] = D + 3      # depth beyond D_max
        depth[3] = -1
        tokens[4, 0] = V + 5  # token out of range
    return B, D, V, dtype, opt, P, Q, tokens, depth, temps


@pytest.mark.parametrize("case", list(STATS_CASES))
def test_verify_stats_outputs_equal_accept_stats(case):
    """The statistics a verification call leaves in its stats_* outputs are
    the bits sv_accept_stats writes afterwards on the call's own depths,
    acceptance rates and accepted lengths (and agree with the oracle's
    statistics of the same inputs)."""
    B, D, V, dtype, opt, P, Q, tokens, depth, temps = _stats_inputs(case)
    Pd, Qd = to_dev(P, dtype), to_dev(Q, dtype)
    tr0, dr0 = padded_offsets(B, D, DEV)
    tok = torch.from_numpy(tokens).to(DEV).reshape(B, D)
    dep = torch.from_numpy(depth).to(DEV)
    T = torch.from_numpy(temps).to(DEV)
    v = sv.Verifier(B, D, V, DEV, alpha=opt.get("alpha", True), stats=True)
    if "shard" in opt:
        W = opt["shard"]

        def shard(rows):  # buffers of W columns at stride W, the last one narrower
            out = []
            for c in range(0, V, W):
                buf = torch.full((rows.shape[0], W), float("nan"), dtype=dtype, device=DEV)
                part = rows[:, c:min(c + W, V)]
                buf[:, :part.shape[1]] = part
                out.append(buf)
            return out

        v.prepare_sharded(shard(Pd), shard(Qd), W, tr0, dr0, tok, dep, T, seed=5, step=2)
    else:
        v.prepare(Pd, Qd, tr0, dr0, tok, dep, T, seed=5, step=2, flags=opt.get("flags", 0))
    for s in v.out.stats.values():
        s.fill_(float("nan"))
    out = v.run(noalloc=opt.get("noalloc", False))
    ref = sv.accept_stats(dep, out.alpha, out.accepted_len, D)
    torch.cuda.synchronize()
    n = 3 * D
    assert torch.equal(out.stats["expected_len"], ref["expected_len"])
    assert torch.equal(out.stats["per_depth"][:n], ref["per_depth"][:n])
    assert torch.equal(out.stats["summary"], ref["summary"])
    if opt.get("invalid"):
        assert np.all(out.accepted_len.cpu().numpy()[1:5] == 0)
    alpha = out.alpha.cpu().numpy().astype(np.float64) if out.alpha is not None else None
    o = oracle.accept_stats(depth, alpha, out.accepted_len.cpu().numpy(), D)
    g = {k: t.cpu().numpy() for k, t in out.stats.items()}
    assert np.allclose(g["expected_len"], o["expected_len"], rtol=1e-5, atol=1e-6)
    assert np.allclose(g["per_depth"][:n].reshape(3, D), o["per_depth"], rtol=1e-5, atol=1e-6)
    assert np.allclose(g["summary"], o["summary"], rtol=1e-5)


@pytest.mark.parametrize("name", ["c4full", "c5"])
def test_verify_stats_outputs_full_batch(name):
    """The same at the two full batch sizes (64 x 16 at V = 151936 bf16 and
    V = 262144 fp32, mixed temperatures on the second), depths from the
    budget as the verification step uses them."""
    w = synth.make(name, device=DEV)
    B, D, V = w.B, w.D, w.V
    bud = sv.allocate_budget(w.conf.to(DEV), w.K)
    v = sv.Verifier(B, D, V, DEV, stats=True)
    v.prepare(w.target.reshape(B * (D + 1), V), w.draft.reshape(B * D, V),
              bud["target_row0"], bud["draft_row0"], w.draft_tokens, bud["depth"],
              w.temperature, seed=11, step=1)
    out = v.run()
    ref = sv.accept_stats(bud["depth"], out.alpha, out.accepted_len, D)
    torch.cuda.synchronize()
    for k in ("expected_len", "per_depth", "summary"):
        assert torch.equal(out.stats[k], ref[k]), k


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("row_pass", ["team", "stream"])
def test_extreme_logit_ranges(dtype, row_pass):
    """Rows whose logits span hundreds of units at full vocabulary: spikes of
    +150..+300 placed in different slices of a row, one slice far below the
    rest, and temperatures 0.3 and 1.  Partial states of such rows differ by
    far more than the float32 range, so every merge (in the row pass and in
    the accept kernel) has to rescale against the true maximum."""
    rng = np.random.default_rng(4242)
    B, D, V = 4, 3, 151936
    temps = np.array([0.3, 1.0, 0.3, 1.0], np.float32)
    P, Q, tokens = random_batch(rng, B, D, V, V, dtype, temps, scale=3.0, noise=1.0)
    for i in range(P.shape[0]):
        j = int(rng.integers(0, V))
        P[i, j] += float(rng.uniform(150.0, 300.0))
        lo = int(rng.integers(0, V - 20000))
        P[i, lo:lo + 20000] -= 200.0
    for i in range(Q.shape[0]):
        j = int(rng.integers(0, V))
        Q[i, j] += float(rng.uniform(150.0, 300.0))
    # drafts that sometimes hit the spikes
    for r in range(B):
        for k in range(D):
            if rng.random() < 0.5:
                tokens[r, k] = int(np.argmax(Q[r * D + k]))
    Pd, Qd = to_dev(P, dtype), to_dev(Q, dtype)
    depth = np.full(B, D, np.int32)
    tr0, dr0 = padded_offsets(B, D, DEV)
    g = gpu_verify(Pd, Qd, tr0, dr0, torch.from_numpy(tokens).to(DEV),
                   torch.from_numpy(depth).to(DEV), torch.from_numpy(temps).to(DEV), seed=9,
                   flags=sv.SV_FLAG_STREAMING_ROW_PASS if row_pass == "stream" else 0)
    Ph = Pd.float().cpu().numpy()
    Qh = Qd.float().cpu().numpy()
    o = oracle_verify(Ph, Qh, tr0.cpu().numpy(), dr0.cpu().numpy(), tokens, depth, temps,
                      np.arange(B), seed=9)
    rep = compare(g, o, np.arange(B), temps, depth, check_flag_rate=False)
    assert rep["mismatched"] == 0 or rep["flagged"] >= rep["mismatched"]
    assert np.all(g["bits"] & sv.BIT_SYNC_TIMEOUT == 0)


@pytest.mark.parametrize("row_pass", ["team", "stream"])
def test_long_fp32_rows_low_temperature(row_pass):
    """fp32 rows of 262144 columns at T = 0.3 and 0.6 with a spike: the
    softmax normaliser is accumulated over 16 groups per thread on the
    streaming pass, against references m log2(e)/T near 60-100, so any
    mismatch between the rounded reference a group's exponentials use and the
    one its rescale assumes compounds group after group (that slip once gave
    alpha errors of 4e-5 here).  alpha must stay within 1e-5 relative."""
    rng = np.random.default_rng(31)
    B, D, V = 4, 2, 262144
    temps = np.array([0.3, 0.3, 0.6, 0.6], np.float32)
    P = (3.0 * rng.standard_normal((B * (D + 1), V))).astype(np.float32)
    for i in range(P.shape[0]):
        P[i, int(rng.integers(0, V))] += 12.0
    Q = np.empty((B * D, V), np.float32)
    for r in range(B):
        for k in range(D):
            Q[r * D + k] = P[r * (D + 1) + k] + rng.standard_normal(V).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, D)).astype(np.int32)
    depth = np.full(B, D, np.int32)
    Pd, Qd = to_dev(P, torch.float32), to_dev(Q, torch.float32)
    tr0, dr0 = padded_offsets(B, D, DEV)
    g = gpu_verify(Pd, Qd, tr0, dr0, torch.from_numpy(tokens).to(DEV),
                   torch.from_numpy(depth).to(DEV), torch.from_numpy(temps).to(DEV), seed=5,
                   flags=sv.SV_FLAG_STREAMING_ROW_PASS if row_pass == "stream" else 0)
    o = oracle_verify(P, Q, tr0.cpu().numpy(), dr0.cpu().numpy(), tokens, depth, temps,
                      np.arange(B), seed=5)
    rep = compare(g, o, np.arange(B), temps, depth, check_flag_rate=False)
    assert rep["mismatched"] == 0 or rep["flagged"] >= rep["mismatched"]


@pytest.mark.parametrize("row_pass", ["team", "stream"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_large_references_low_temperature(dtype, row_pass):
    """Peaked rows at T = 0.1 .. 0.6 whose peak (about 40 above the bulk) the
    draft rows share, so p / q and alpha are near 1 and the references
    m log2(e)/T reach 230 .. 750, where one float32 ulp is 1.5e-5 .. 6e-5.
    Every normaliser, rescale and exponential must use the same rounded
    reference fl(m sl) (its rounding then cancels): mixing in the exact
    product once gave alpha errors of 1e-5 and more here.  alpha within 1e-5
    relative, tokens outside the oracle's flag bands, and draft confidences
    within 1e-5 relative."""
    rng = np.random.default_rng(43)
    B, D, V = 4, 3, 151936
    temps = np.array([0.3, 0.2, 0.1, 0.6], np.float32)
    P = (3.0 * rng.standard_normal((B * (D + 1), V))).astype(np.float32)
    peaks = rng.integers(0, V, size=P.shape[0])
    for i in range(P.shape[0]):
        P[i, peaks[i]] = 40.0 + 12.0 * rng.random()
    Q = np.empty((B * D, V), np.float32)
    for r in range(B):
        for k in range(D):
            Q[r * D + k] = P[r * (D + 1) + k] + 0.02 * rng.standard_normal(V).astype(np.float32)
    Pd, Qd = to_dev(P, dtype), to_dev(Q, dtype)
    Ph, Qh = Pd.float().cpu().numpy(), Qd.float().cpu().numpy()
    tokens = np.array([[peaks[r * (D + 1) + k] for k in range(D)] for r in range(B)], np.int32)
    tokens[1, 2] = (tokens[1, 2] + 1) % V  # one draft off the peak
    depth = np.full(B, D, np.int32)
    tr0, dr0 = padded_offsets(B, D, DEV)
    tok_d, temps_d = torch.from_numpy(tokens).to(DEV), torch.from_numpy(temps).to(DEV)
    g = gpu_verify(Pd, Qd, tr0, dr0, tok_d, torch.from_numpy(depth).to(DEV), temps_d, seed=9,
                   flags=sv.SV_FLAG_STREAMING_ROW_PASS if row_pass == "stream" else 0)
    o = oracle_verify(Ph, Qh, tr0.cpu().numpy(), dr0.cpu().numpy(), tokens, depth, temps,
                      np.arange(B), seed=9)
    rep = compare(g, o, np.arange(B), temps, depth, check_flag_rate=False)
    assert rep["mismatched"] == 0 or rep["flagged"] >= rep["mismatched"]
    conf = sv.draft_confidence(Qd, dr0, tok_d, temps_d).cpu().numpy().astype(np.float64)
    ref = oracle.draft_confidence(Qh, dr0.cpu().numpy(), tokens, temps)
    assert np.all(np.abs(conf - ref) <= 1e-5 * ref + 1e-30), (conf, ref)
    assert ref[0, 0] > 0.5  # the peaks decide: confidences near 1 are checked
