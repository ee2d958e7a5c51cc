"""The C ABI library loads and exports every entry point include/specverify.h
declares; argument validation (which runs before any HIP call) returns the
documented status codes.  No compute call is made: this runs without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


@pytest.fixture(scope="module")
def sv():
    from lossless_draft_verification_softmax_amd import specverify
    if not os.path.exists(specverify.LIB_PATH):
        from lossless_draft_verification_softmax_amd import build
        build.build()
    return specverify


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(sv):
    lib = sv.load()
    names = declared_functions()
    assert set(names) == set(sv.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings_and_version(sv):
    assert sv.status_string(0) == "ok"
    assert "workspace" in sv.status_string(3)
    assert "gfx950" in sv.load().sv_version().decode()


def test_k_rho_matches_equation(sv):
    path = os.path.join(ROOT, "tests", "golden", "k_rho.txt")
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            B, D, rho, K = line.split()
            assert sv.k_rho(int(B), int(D), float(rho)) == int(K)
    assert sv.k_rho(-1, 3, 0.5) == -1
    assert sv.k_rho(4, 3, 1.5) == -1


def test_workspace_bytes(sv):
    assert sv.workspace_bytes(64, 16, 151936) > 0
    assert sv.workspace_bytes(64, 16, 151936) % 256 == 0
    assert sv.workspace_bytes(64, 65, 151936) == 0
    assert sv.workspace_bytes(-1, 3, 10) == 0
    assert sv.workspace_bytes(4, 3, 0) == 0


def test_noalloc_scratch_limits(sv):
    # the batch sizes the header states for the no-allocation entry point's
    # 32 MiB array: the largest B at D_max = 16 fits, one more does not
    lim = sv.SV_NOALLOC_SCRATCH_BYTES
    for B, V in ((354, 262144), (426, 151936)):
        assert sv.workspace_bytes(B, 16, V) <= lim
        assert sv.workspace_bytes(B + 1, 16, V) > lim


def _args(sv, **kw):
    a = sv.SvVerifyArgs()
    a.dtype = sv.SV_DTYPE_BF16
    a.B, a.D_max, a.V, a.row_stride = 2, 3, 64, 64
    fake = 1 << 20  # 16-byte aligned, never dereferenced: validation fails first
    for f in ("target_logits", "target_row0", "draft_logits", "draft_row0", "draft_tokens",
              "depth", "temperature", "accepted_len", "out_tokens", "num_out"):
        setattr(a, f, fake)
    a.workspace = fake
    a.workspace_bytes = 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def call(sv, a):
    return sv.load().sv_verify_batch(ctypes.byref(a), None)


def test_verify_validation_codes(sv):
    lib = sv.load()
    assert lib.sv_verify_batch(None, None) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(sv, _args(sv, B=-1)) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(sv, _args(sv, D_max=65)) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(sv, _args(sv, V=0)) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(sv, _args(sv, row_stride=32)) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(sv, _args(sv, dtype=7)) == sv.SV_ERR_UNSUPPORTED
    assert call(sv, _args(sv, flags=16)) == sv.SV_ERR_UNSUPPORTED
    # a known flag passes validation (the too-small workspace is caught next)
    assert call(sv, _args(sv, flags=sv.SV_FLAG_TEAM_WAIT_GIVE_UP)) == sv.SV_ERR_WORKSPACE_TOO_SMALL
    assert call(sv, _args(sv, target_logits=None)) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(sv, _args(sv, draft_row0=None)) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(sv, _args(sv, target_logits=(1 << 20) + 2)) == sv.SV_ERR_UNSUPPORTED
    assert call(sv, _args(sv, V=60, row_stride=60)) == sv.SV_ERR_UNSUPPORTED
    assert call(sv, _args(sv, workspace=None)) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(sv, _args(sv, workspace=(1 << 20) + 16)) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(sv, _args(sv)) == sv.SV_ERR_WORKSPACE_TOO_SMALL
    assert call(sv, _args(sv, B=0)) == sv.SV_OK  # empty batch: nothing to do


def test_budget_and_stats_validation_codes(sv):
    lib = sv.load()
    fake = 1 << 20
    assert lib.sv_allocate_budget(fake, -1, 3, None, 4, fake, None, None, None, None) == 1
    assert lib.sv_allocate_budget(fake, 64, 65, None, 4, fake, None, None, None, None) == 1
    assert lib.sv_allocate_budget(fake, 5000, 0, None, 4, fake, None, None, None, None) == 1
    assert lib.sv_allocate_budget(None, 4, 3, None, 4, fake, None, None, None, None) == 1
    assert lib.sv_allocate_budget(fake, 4, 3, None, 4, None, None, None, None, None) == 1
    assert lib.sv_allocate_budget(fake, 0, 3, None, 4, None, None, None, None, None) == 0
    assert lib.sv_accept_stats(fake, None, fake, 4, 65, None, None, None, None) == 1
    assert lib.sv_accept_stats(None, None, fake, 4, 3, None, None, None, None) == 1
    assert lib.sv_accept_stats(None, None, None, 0, 3, None, None, None, None) == 0


def test_confidence_validation_codes(sv):
    lib = sv.load()
    fake = 1 << 20  # a 256-byte aligned fake device address; nothing is dereferenced
    ws = lib.sv_draft_confidence_workspace_bytes(0, 64, 16, 151936)
    assert ws == 64 * 16 * 10 * 4 * 8  # 10 segments of 2048 vectors, a float2 per wavefront
    assert lib.sv_draft_confidence_workspace_bytes(0, 0, 16, 100) == 256
    assert lib.sv_draft_confidence_workspace_bytes(7, 4, 4, 100) == 0
    assert lib.sv_draft_confidence_workspace_bytes(1, 4, 4, 0) == 0

    def call(dtype=0, B=4, D=3, V=1000, stride=1000, logits=fake, row0=fake, tok=fake, dep=None,
             T=fake, conf=fake, ws_ptr=fake, ws_bytes=1 << 20):
        return lib.sv_draft_confidence(dtype, B, D, V, stride, logits, row0, tok, dep, T, conf,
                                       ws_ptr, ws_bytes, None)

    assert call(dtype=5) == sv.SV_ERR_UNSUPPORTED
    assert call(B=-1) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(stride=999) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(B=0) == sv.SV_OK
    assert call(D=0) == sv.SV_OK
    assert call(logits=None) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(tok=None) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(logits=fake + 4) == sv.SV_ERR_UNSUPPORTED
    assert call(stride=1004) == sv.SV_ERR_UNSUPPORTED      # not a multiple of 8 bf16 elements
    assert call(ws_ptr=fake + 16) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(ws_bytes=8) == sv.SV_ERR_WORKSPACE_TOO_SMALL


def test_ratio_validation_codes(sv):
    lib = sv.load()
    fake = 1 << 20
    D = ctypes.c_double
    I = ctypes.c_int32
    F = ctypes.c_float

    def call(B=4, Dm=3, ratios=(0.25, 0.5), tb=(4,), tl=(1.0, 2.0), choice=fake, conf=fake):
        r = (D * len(ratios))(*ratios) if ratios is not None else None
        return lib.sv_select_budget_ratio(conf, B, Dm, None, len(ratios or ()), r, len(tb),
                                          (I * len(tb))(*tb), (F * len(tl))(*tl), choice, fake,
                                          None, fake, None, None, None, None)

    assert call(B=0) == sv.SV_OK
    assert call(B=-1) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(B=100, Dm=64) == sv.SV_ERR_INVALID_ARGUMENT   # over SV_MAX_BUDGET_POSITIONS
    assert call(ratios=()) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(ratios=(0.5,) * 9, tl=(1.0,) * 9) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(ratios=(0.5, 1.5)) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(tb=(4, 4), tl=(1.0, 2.0, 1.0, 2.0)) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(tl=(1.0, 0.0)) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(tl=(1.0, float("inf"))) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(choice=None) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(conf=None) == sv.SV_ERR_INVALID_ARGUMENT


def test_sample_validation_codes(sv):
    lib = sv.load()
    fake = 1 << 20

    def call(dtype=0, B=4, V=100, stride=100, logits=fake, base=0, idx=fake, istride=1, T=fake,
             tok=fake, tstride=1):
        return lib.sv_sample_rows(dtype, B, V, stride, logits, base, idx, istride, T, None, 0, 0,
                                  0, tok, tstride, None)

    assert call(dtype=3) == sv.SV_ERR_UNSUPPORTED
    assert call(B=0) == sv.SV_OK
    assert call(B=-1) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(V=0) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(stride=99) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(base=-1) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(istride=-1) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(tstride=0) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(logits=None) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(idx=None) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(tok=None) == sv.SV_ERR_INVALID_ARGUMENT


def test_sharded_verify_validation_codes(sv):
    lib = sv.load()
    fake = 1 << 20
    P = ctypes.c_void_p

    def call(n=2, w=64, V=120, shards=(fake, fake + 4096), dshards=None, stride=64, B=1,
             draft_row0=None):
        a = sv.SvVerifyArgs()
        a.dtype, a.B, a.D_max, a.V, a.row_stride = 0, B, 3, V, stride
        a.target_row0, a.depth, a.temperature = fake, fake, fake
        a.accepted_len, a.out_tokens, a.num_out, a.draft_tokens = fake, fake, fake, fake
        a.draft_row0 = draft_row0
        a.workspace, a.workspace_bytes = fake, 1 << 30
        t = (P * len(shards))(*shards) if shards is not None else None
        d = (P * len(dshards))(*dshards) if dshards is not None else None
        return lib.sv_verify_batch_sharded(ctypes.byref(a), n, w, t, d, None)

    assert call(shards=None) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(n=0) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(n=17) == sv.SV_ERR_INVALID_ARGUMENT
    assert call(w=60) == sv.SV_ERR_UNSUPPORTED             # not a multiple of 8
    assert call(n=3, shards=(fake, fake, fake)) == sv.SV_ERR_INVALID_ARGUMENT  # ceil(120/64) = 2
    assert call(shards=(fake, fake + 8)) == sv.SV_ERR_INVALID_ARGUMENT         # misaligned shard
    assert call(stride=60) == sv.SV_ERR_INVALID_ARGUMENT   # stride below the shard width
    assert call(dshards=(fake, fake)) == sv.SV_ERR_INVALID_ARGUMENT            # no draft_row0
    assert call(B=0) == sv.SV_OK


def test_noalloc_and_stream_read_validation_codes(sv):
    lib = sv.load()
    fake = 1 << 20
    # sizes whose workspace exceeds the static scratch: rejected on the host
    big = _args(sv, B=4096, D_max=64, V=262144, row_stride=262144)
    assert lib.sv_verify_batch_noalloc(ctypes.byref(big), None) == sv.SV_ERR_SCRATCH_TOO_SMALL
    assert lib.sv_verify_batch_noalloc(None, None) == sv.SV_ERR_INVALID_ARGUMENT
    assert "scratch" in sv.status_string(sv.SV_ERR_SCRATCH_TOO_SMALL)
    sink = fake
    assert lib.sv_stream_read(None, 1024, 4, sink, None) == sv.SV_ERR_INVALID_ARGUMENT
    assert lib.sv_stream_read(fake + 4, 1024, 4, sink, None) == sv.SV_ERR_INVALID_ARGUMENT
    assert lib.sv_stream_read(fake, 1000, 4, sink, None) == sv.SV_ERR_INVALID_ARGUMENT
    assert lib.sv_stream_read(fake, 1024, 0, sink, None) == sv.SV_ERR_INVALID_ARGUMENT
    assert lib.sv_stream_read(fake, 1024, 33, sink, None) == sv.SV_ERR_INVALID_ARGUMENT
    assert lib.sv_stream_read(fake, 1024, 4, None, None) == sv.SV_ERR_INVALID_ARGUMENT
    assert lib.sv_stream_read(fake, 0, 4, sink, None) == sv.SV_OK


def _c_layout(struct, fields):
    """sizeof and offsetof of a header struct, from a C program built with gcc."""
    import subprocess
    import tempfile
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "specverify.h"',
             'int main(void) {', f'  printf("%zu\\n", sizeof({struct}));']
    lines += [f'  printf("%zu\\n", offsetof({struct}, {f}));' for f in fields]
    lines += ['  return 0;', '}']
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        open(src, "w").write("\n".join(lines) + "\n")
        subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), src, "-o", exe],
                       check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    return [int(x) for x in out]


@pytest.mark.parametrize("name", ["SvVerifyArgs", "SvDiag"])
def test_binding_struct_layout_matches_header(sv, name):
    cls = getattr(sv, name)
    struct = {"SvVerifyArgs": "sv_verify_args", "SvDiag": "sv_diag"}[name]
    fields = [f[0] for f in cls._fields_]
    c = _c_layout(struct, fields)
    assert c[0] == ctypes.sizeof(cls)
    assert c[1:] == [getattr(cls, f).offset for f in fields]
