"""GPU parity of greedy (T = 0) verification on constructed full-vocabulary
rows: the arg max must be the first maximal column (ties to the lowest
index, -0 equal to +0, as torch.argmax's first-occurrence rule), and rows
holding NaN, +inf or only -inf must mark their request invalid.  Each row
pattern puts the deciding columns where the row pass splits its work: in
different team members' slices, at slice boundaries, in both 16-byte
vectors of a thread, at the first and the last column, and (for a row
length that is not a multiple of 8) in the ragged tail.  Expected values
come from the oracle on the same (rounded) logits."""
import numpy as np
import pytest
import torch

from lossless_draft_verification_softmax_amd import specverify as sv
from tests.parity import compare, gpu_verify, oracle_verify, padded_offsets

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 2
SLICE = 15200  # columns per team member at V = 151936 bf16


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sv.load()


def negative_row(rng, V):
    return -np.abs(3.0 * rng.standard_normal(V)).astype(np.float32) - 0.5


def normal_row(rng, V):
    return (3.0 * rng.standard_normal(V)).astype(np.float32)


def build(rng, V):
    """Target rows [B * (D + 1), V]; request r owns rows 3r .. 3r + 2."""
    rows = []
    # r0: maximum +0 after an earlier -0 (the -0 wins), -0 alone, spread ties
    a = negative_row(rng, V)
    a[2 * SLICE + 17] = -0.0
    a[7 * SLICE + 3] = 0.0
    b = negative_row(rng, V)
    for c in (SLICE + 1, 3 * SLICE + 8, 9 * SLICE + 2):
        b[min(c, V - 1)] = -0.0
    c_ = normal_row(rng, V)
    c_[rng.choice(V, size=24, replace=False)] = 40.0
    rows += [a, b, c_]
    # r1: maximum at the last column, at column 0, ties on slice boundaries
    a = normal_row(rng, V)
    a[V - 1] = 40.0
    b = normal_row(rng, V)
    b[0] = 40.0
    c_ = normal_row(rng, V)
    for m in range(1, 10):
        for col in (m * SLICE - 1, m * SLICE):
            if col < V:
                c_[col] = 40.0
    rows += [a, b, c_]
    # r2: a NaN inside one member's slice of the middle row
    a, b, c_ = normal_row(rng, V), normal_row(rng, V), normal_row(rng, V)
    b[4 * SLICE + 77] = np.nan
    rows += [a, b, c_]
    # r3: a row of -inf only
    a, b, c_ = normal_row(rng, V), normal_row(rng, V), normal_row(rng, V)
    a[:] = -np.inf
    rows += [a, b, c_]
    # r4: +inf in the last row
    a, b, c_ = normal_row(rng, V), normal_row(rng, V), normal_row(rng, V)
    c_[6 * SLICE + 5] = np.inf
    rows += [a, b, c_]
    # r5: plain rows; r6: -inf everywhere but a few columns (masked vocabulary)
    rows += [normal_row(rng, V) for _ in range(3)]
    m = []
    for _ in range(3):
        x = np.full(V, -np.inf, np.float32)
        x[rng.choice(V, size=5, replace=False)] = rng.normal(0, 1, 5).astype(np.float32)
        m.append(x)
    rows += m
    # r7: maxima in the last (ragged) columns, or the last whole vector
    a, b, c_ = normal_row(rng, V), normal_row(rng, V), normal_row(rng, V)
    a[V - 3] = 40.0
    b[V - 9] = 40.0
    b[V - 2] = 40.0
    c_[V - 8] = 39.0
    rows += [a, b, c_]
    return np.stack(rows)


@pytest.mark.parametrize("row_pass", ["team", "stream"])
@pytest.mark.parametrize("V", [151936, 151931])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_greedy_argmax_edge_rows(dtype, V, row_pass):
    rng = np.random.default_rng(7 + V % 13)
    P = build(rng, V)
    B = P.shape[0] // (D + 1)
    stride = (V + 7) // 8 * 8  # 16-byte aligned rows; padding is NaN and never read
    Pp = np.full((P.shape[0], stride), np.nan, np.float32)
    Pp[:, :V] = P
    Pd = torch.from_numpy(Pp).to(DEV).to(dtype)
    Ph = np.ascontiguousarray(Pd.float().cpu().numpy()[:, :V])
    # drafts equal to the first arg max of rows 0 and 1, so every request
    # that is valid emits the arg max of all three rows
    tokens = np.zeros((B, D), np.int32)
    for r in range(B):
        for k in range(D):
            row = Ph[r * (D + 1) + k]
            tokens[r, k] = int(np.argmax(np.where(np.isnan(row), -np.inf, row)))
    depth = np.full(B, D, np.int32)
    temps = np.zeros(B, np.float32)
    tr0, dr0 = padded_offsets(B, D, DEV)
    flags = sv.SV_FLAG_STREAMING_ROW_PASS if row_pass == "stream" else 0
    g = gpu_verify(Pd, None, tr0, dr0, torch.from_numpy(tokens).to(DEV),
                   torch.from_numpy(depth).to(DEV), torch.from_numpy(temps).to(DEV), flags=flags,
                   V=V)
    o = oracle_verify(Ph, None, tr0.cpu().numpy(), None, tokens, depth, temps, np.arange(B))
    compare(g, o, np.arange(B), temps, depth, check_alpha=False, check_flag_rate=False)
    # the patterns above decide: valid requests accept both drafts
    valid = [0, 1, 5, 6, 7]
    assert np.all(g["bits"][[2, 3, 4]] & sv.BIT_BAD_ROW)
    assert np.all(g["accepted_len"][valid] == D)
    assert g["out_tokens"][0, 0] == 2 * SLICE + 17          # -0 before +0
    assert g["out_tokens"][1, 2] == SLICE - 1               # first boundary tie
    assert g["out_tokens"][1, 0] == V - 1 and g["out_tokens"][1, 1] == 0
