"""sv_verify_batch_noalloc (the entry point for callers that cannot allocate:
static device scratch instead of a workspace) against sv_verify_batch, both
through the C ABI, on two calls in a row, the second on a smaller batch.  The
two share their kernels, so every output must agree bit for bit; the first
batch is also held against the CPU oracle."""
import ctypes

import numpy as np
import pytest
import torch

from lossless_draft_verification_softmax_amd import specverify as sv
from lossless_draft_verification_softmax_amd import synth
from tests.parity import compare, host_f32, oracle_verify, padded_offsets

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
    # ragged depths, every request at least one position short of full
    g = torch.Generator().manual_seed(seed)
    depth = torch.randint(0, w.D + 1, (w.B,), generator=g, dtype=torch.int32).to(DEV)
    return w, tr0, dr0, depth


def _outputs(v):
    o = v.out
    return {k: getattr(o, k).clone() for k in ("accepted_len", "out_tokens", "num_out", "alpha",
                                               "diag")}


def _run_both(w, tr0, dr0, depth, seed):
    ref = sv.Verifier(w.B, w.D, w.V, DEV, alpha=True, diag=True)
    ref.prepare(w.target, w.draft, tr0, dr0, w.draft_tokens, depth, w.temperature, seed=seed)
    na = sv.Verifier(w.B, w.D, w.V, DEV, alpha=True, diag=True)
    na.prepare(w.target, w.draft, tr0, dr0, w.draft_tokens, depth, w.temperature, seed=seed)
    # Poison the outputs of the no-allocation call and drop its workspace from
    # the argument block: the entry point must ignore it.
    for t in (na.out.accepted_len, na.out.out_tokens, na.out.num_out, na.out.diag):
        t.fill_(-7)
    na.out.alpha.fill_(float("nan"))
    na.args.workspace = None
    na.args.workspace_bytes = 0
    ref.run()
    st = sv.load().sv_verify_batch_noalloc(ctypes.byref(na.args), sv._stream(torch.device(DEV)))
    assert st == sv.SV_OK, sv.status_string(st)
    torch.cuda.synchronize()
    a, b = _outputs(ref), _outputs(na)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    return a


def test_noalloc_matches_verify_batch_two_calls():
    # first call: mixed temperatures over several team tiles and a ragged tail
    w1, tr1, dr1, dep1 = _case("c5", B=24, V=40000, seed=1)
    print(f"noalloc call 1: B={w1.B} D={w1.D} V={w1.V} {w1.target.dtype}", flush=True)
    out1 = _run_both(w1, tr1, dr1, dep1, seed=3)
    # the first batch is also held against the oracle
    th, dh = host_f32(w1.target).reshape(-1, w1.V), host_f32(w1.draft).reshape(-1, w1.V)
    temps = w1.temperature.cpu().numpy()
    reqs = np.arange(w1.B)
    o = oracle_verify(th, dh, tr1.cpu().numpy(), dr1.cpu().numpy(), w1.draft_tokens.cpu().numpy(),
                      dep1.cpu().numpy(), temps, reqs, seed=3)
    g = dict(accepted_len=out1["accepted_len"].cpu().numpy(),
             out_tokens=out1["out_tokens"].cpu().numpy(),
             num_out=out1["num_out"].cpu().numpy(), alpha=out1["alpha"].cpu().numpy(),
             bits=out1["diag"][:, 2].cpu().numpy().astype(np.uint32))
    compare(g, o, reqs, temps, dep1.cpu().numpy())
    # second call: a smaller bf16 batch, on the scratch the first call left
    w2, tr2, dr2, dep2 = _case("c2", B=5, V=1000, seed=2)
    print(f"noalloc call 2: B={w2.B} D={w2.D} V={w2.V} {w2.target.dtype}", flush=True)
    _run_both(w2, tr2, dr2, dep2, seed=4)


def test_noalloc_rejects_batches_beyond_its_scratch():
    a = sv.SvVerifyArgs()
    a.dtype = sv.SV_DTYPE_BF16
    a.B, a.D_max, a.V, a.row_stride = 4096, 64, 262144, 262144
    assert sv.workspace_bytes(4096, 64, 262144) > sv.SV_NOALLOC_SCRATCH_BYTES
    st = sv.load().sv_verify_batch_noalloc(ctypes.byref(a), None)
    assert st == sv.SV_ERR_SCRATCH_TOO_SMALL
