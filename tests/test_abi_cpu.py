"""The C ABI library loads and exports every symbol include/kda.h declares, and
rejects bad arguments before launching anything (no GPU needed)."""
import os
import re

import pytest

import gated_delta_rule_76_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_symbols():
    syms = set()
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            txt = open(os.path.join(inc, f)).read()
            syms |= set(re.findall(r"^KDA_API\s+[\w\s\*]*?\b(\w+)\s*\(", txt, re.M))
    return sorted(syms)


def test_header_declares_the_abi():
    assert _header_symbols() == sorted(kda.ABI_SYMBOLS)


def test_library_exports_every_declared_symbol():
    assert os.path.exists(kda.library_path())
    assert sorted(kda.exported_symbols()) == _header_symbols()


def test_checked_build_exports_the_same_abi():
    """libkda_checked.so (bounds checks in the kernels) is built beside
    libkda.so and exports every declared symbol; each reports which it is."""
    assert os.path.exists(kda.CHECKED_LIB_PATH)
    try:
        assert kda.select_build(checked=True) == kda.CHECKED_LIB_PATH
        assert sorted(kda.exported_symbols()) == _header_symbols()
        assert kda.build_checked() is True
        assert kda.check_sites() == 0
    finally:
        assert kda.select_build(checked=False) == kda.LIB_PATH
    assert kda.build_checked() is False
    assert kda.check_sites() == 0


def test_version_and_status_strings():
    assert kda.version() == 1
    for code, name in kda.STATUS.items():
        assert kda.status_string(code) == name
    assert kda.status_string(99) == "KDA_ERR_UNKNOWN"


def test_wait_limit_hook():
    default = kda.wait_limit()
    assert default == 1 << 24
    try:
        assert kda.set_wait_limit(-1) == 1          # KDA_ERR_INVALID_ARG
        assert kda.wait_limit() == default
        assert kda.set_wait_limit(0) == 0 and kda.wait_limit() == 0
    finally:
        assert kda.set_wait_limit(default) == 0
    assert kda.wait_limit() == default


def test_ring_cap_hook():
    ws = kda.lib().kda_fwd_chunked_workspace_bytes
    one = ws(1, 64, 1, 128, 128, 64, kda.KDA_BF16)
    assert kda.ring_cap() == 512 << 20
    try:
        kda.set_ring_cap(3 * one)           # room for one chunk of one chain per ring buffer
        assert kda.ring_cap() == 3 * one
        assert ws(1, 64, 1, 128, 128, 64, kda.KDA_BF16) == one            # one chunk: no ring
        assert ws(1, 640, 1, 128, 128, 64, kda.KDA_BF16) == 2 * one + 128 * 128 * 4
        assert ws(2, 640, 1, 128, 128, 64, kda.KDA_BF16) == 4 * one + 2 * 128 * 128 * 4
    finally:
        kda.set_ring_cap(0)
    assert kda.ring_cap() == 512 << 20


def test_workspace_query():
    ws = kda.lib().kda_fwd_chunked_workspace_bytes
    one = ws(1, 64, 1, 128, 128, 64, kda.KDA_BF16)      # one chunk's slot
    assert one % 1024 == 0 and 60 * 1024 <= one <= 62 * 1024
    assert ws(1, 65, 1, 128, 128, 64, kda.KDA_BF16) == 2 * one   # ragged tail: one more slot
    assert ws(4, 4096, 16, 128, 128, 64, kda.KDA_BF16) == 4 * 16 * 64 * one  # fits: no ring
    # Past the 512 MiB slot budget the sequence runs in segments through two
    # ring buffers plus a carrier state: the size stops growing with T.
    cap, state = 512 << 20, 4 * 16 * 128 * 128 * 4
    big = ws(4, 16384, 16, 128, 128, 64, kda.KDA_BF16)
    assert big == 2 * 64 * 64 * one + state                     # 4 segments of 64 chunks
    assert big <= cap + state
    assert ws(4, 1 << 20, 16, 128, 128, 64, kda.KDA_BF16) <= cap + state
    assert ws(1, 1 << 22, 16, 128, 128, 64, kda.KDA_BF16) <= cap + 16 * 128 * 128 * 4
    assert ws(1, 0, 1, 128, 128, 64, kda.KDA_BF16) == 0
    assert ws(1, 64, 1, 128, 128, 64, kda.KDA_F32) == 0          # unsupported combination
    assert ws(1, 64, 1, 48, 128, 64, kda.KDA_BF16) == 0


# Fake but 16-byte-aligned addresses: every call below must fail validation
# before any launch, so nothing is ever dereferenced.
P = 0x100000


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, alpha=P, beta=P, S0=None, o=P, S_T=P, B=1, T=64, H=1, d_k=64,
             d_v=64, chunk=64, dtype=kda.KDA_BF16, ws=None, ws_bytes=0)
    a.update(kw)
    return kda.kda_fwd_chunked_raw(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"], a["o"],
                                   a["S_T"], a["B"], a["T"], a["H"], a["d_k"], a["d_v"], a["chunk"],
                                   a["dtype"], a["ws"], a["ws_bytes"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(alpha=None), 1),
    (dict(beta=None), 1), (dict(o=None), 1),
    (dict(B=0), 1), (dict(H=0), 1), (dict(T=-1), 1), (dict(dtype=7), 1),
    (dict(q=P + 8), 1), (dict(o=P + 4), 1), (dict(S0=P + 4), 1), (dict(S_T=P + 2), 1),
    (dict(beta=P + 1), 1),
    (dict(d_k=48), 2), (dict(d_v=256), 2), (dict(chunk=128), 2), (dict(chunk=8), 2),
    (dict(dtype=kda.KDA_F32, d_k=128, chunk=64), 2),
])
def test_fwd_validation(kw, code):
    assert _fwd(**kw) == code


def test_fwd_workspace_checks():
    need = kda.lib().kda_fwd_chunked_workspace_bytes(1, 64, 1, 64, 64, 64, kda.KDA_BF16)
    assert need > 0
    assert _fwd() == 3                                   # no workspace
    assert _fwd(ws=P, ws_bytes=need - 1) == 3            # too small
    assert _fwd(ws=P + 8, ws_bytes=need) == 3            # misaligned


def test_fwd_t0_without_state_is_a_no_op():
    # T = 0 and no S_T: nothing to do, nothing launched, success.
    assert _fwd(T=0, S_T=None, q=None, k=None, v=None, alpha=None, beta=None, o=None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(S=None), 1), (dict(o=None), 1), (dict(B=0), 1), (dict(S=P + 4), 1),
    (dict(d_k=100), 2), (dict(dtype=3), 1),
])
def test_decode_validation(kw, code):
    a = dict(q=P, k=P, v=P, alpha=P, beta=P, S=P, o=P, B=2, H=2, d_k=128, d_v=128,
             dtype=kda.KDA_BF16)
    a.update(kw)
    assert kda.kda_decode_step_raw(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S"], a["o"],
                                   a["B"], a["H"], a["d_k"], a["d_v"], a["dtype"]) == code


def test_torch_front_end_checks_shapes():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        kda.kda_fwd_chunked(q, q, q, q, torch.zeros(1, 4, 2), None)
    with pytest.raises(TypeError):
        kda.kda_fwd_chunked(q.double(), q.double(), q.double(), q.double(),
                            torch.zeros(1, 4, 1, dtype=torch.float64), None)


def test_package_never_imports_the_oracle():
    import ast
    pkg = os.path.join(ROOT, "gated_delta_rule_76_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                tree = ast.parse(open(os.path.join(dirpath, f)).read())
                for node in ast.walk(tree):
                    if isinstance(node, ast.Import):
                        assert all(not a.name.startswith("oracle") for a in node.names), f
                    if isinstance(node, ast.ImportFrom):
                        assert not (node.module or "").startswith("oracle"), f


@pytest.mark.parametrize("kw,code", [
    (dict(gate=3), 1), (dict(gate=-1), 1), (dict(rule=2), 1),
    (dict(gate=0, alpha=None), 1),               # per-channel gate needs alpha
    (dict(gate=1, alpha=None), 1),               # per-head gate needs alpha
    (dict(gate=1, alpha=P + 1), 1),              # per-head gate: natural alignment
    (dict(gate=0, alpha=P + 2), 1),              # per-channel gate: 16-byte alignment
])
def test_fwd_ex_validation(kw, code):
    a = dict(q=P, k=P, v=P, alpha=P, beta=P, S0=None, o=P, S_T=P, B=1, T=64, H=1, d_k=64,
             d_v=64, chunk=64, dtype=kda.KDA_BF16, ws=None, ws_bytes=0, gate=0, rule=0)
    a.update(kw)
    assert kda.kda_fwd_chunked_raw(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"], a["o"],
                                   a["S_T"], a["B"], a["T"], a["H"], a["d_k"], a["d_v"], a["chunk"],
                                   a["dtype"], a["ws"], a["ws_bytes"], None, a["gate"],
                                   a["rule"]) == code


def test_fwd_ex_gate_none_still_checks_the_workspace():
    # alpha may be NULL without a gate; the call then fails on the missing
    # workspace, before any launch
    assert kda.kda_fwd_chunked_raw(P, P, P, None, P, None, P, P, 1, 64, 1, 64, 64, 64,
                                   kda.KDA_BF16, None, 0, None, 2, 0) == 3


@pytest.mark.parametrize("kw,code", [
    (dict(gate=5), 1), (dict(rule=9), 1), (dict(gate=0, alpha=None), 1),
    (dict(gate=1, alpha=None), 1), (dict(gate=1, alpha=P + 1), 1),
])
def test_decode_ex_validation(kw, code):
    a = dict(q=P, k=P, v=P, alpha=P, beta=P, S=P, o=P, B=2, H=2, d_k=128, d_v=128,
             dtype=kda.KDA_BF16, gate=0, rule=0)
    a.update(kw)
    assert kda.kda_decode_step_raw(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S"], a["o"],
                                   a["B"], a["H"], a["d_k"], a["d_v"], a["dtype"], None,
                                   a["gate"], a["rule"]) == code


def test_torch_front_end_checks_gate_names():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        kda.kda_fwd_chunked(q, q, q, q, torch.zeros(1, 4, 1), None, gate="vector")
    with pytest.raises(ValueError):
        kda.kda_fwd_chunked(q, q, q, q, torch.zeros(1, 4, 1), None, rule="gla")


@pytest.mark.parametrize("kw,code", [
    (dict(c=-0.1), 1), (dict(c=float("nan")), 1), (dict(c=float("inf")), 1),
    (dict(gate=4), 1), (dict(g=None, gate=0), 1),
])
def test_fwd_fused_validation(kw, code):
    a = dict(c=0.1, gate=0, rule=0, g=P)
    a.update(kw)
    assert kda.kda_fwd_chunked_fused_raw(P, P, P, a["g"], P, a["c"], None, P, P, 1, 64, 1, 64, 64,
                                         64, kda.KDA_BF16, a["gate"], a["rule"]) == code


def test_decode_fused_validation():
    assert kda.kda_decode_step_fused_raw(P, P, P, P, P, -1.0, P, P, 2, 2, 128, 128, kda.KDA_BF16,
                                         0, 0) == 1
    assert kda.kda_decode_step_fused_raw(P, P, P, None, P, 0.1, P, P, 2, 2, 128, 128, kda.KDA_BF16,
                                         1, 0) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(L=0), 1), (dict(N=0), 1), (dict(dtype=5), 1),
    (dict(L=2000), 2), (dict(d=12), 2), (dict(d_k=600), 2), (dict(h=P + 8), 1),
    (dict(out=P), 1),                                   # out overlaps the inputs
])
def test_attnres_validation(kw, code):
    a = dict(q=P, k=P + (1 << 24), h=P + (2 << 24), out=P + (3 << 24), L=4, N=8, d_k=16, d=64,
             dtype=kda.KDA_BF16)
    a.update(kw)
    assert kda.attnres_forward_raw(a["q"], a["k"], a["h"], a["out"], a["L"], a["N"], a["d_k"], a["d"],
                                   a["dtype"]) == code


def test_workspace_query_properties():
    """Seeded random sizes: while every chunk's slot fits the 512 MiB budget the
    workspace is exactly one slot per (chain, chunk); past it, two ring
    buffers plus one carried fp32 state per chain, never more than the budget
    plus the carried states, and never less than two chunks' slots for every
    chain (the ring always holds a segment in each half)."""
    import numpy as np
    rng = np.random.Generator(np.random.PCG64(77))
    cap = 512 << 20
    for _ in range(300):
        dtype = [kda.KDA_F32, kda.KDA_BF16][rng.integers(2)]
        dk, dv = int(rng.choice([16, 32, 64, 128])), int(rng.choice([16, 32, 64, 128]))
        C = int(rng.choice([16, 32, 64]))
        B, H = int(rng.integers(1, 9)), int(rng.integers(1, 33))
        T = int(rng.integers(0, 1 << 18))
        slot = kda.workspace_bytes(1, C, 1, dk, dv, C, dtype)
        got = kda.workspace_bytes(B, T, H, dk, dv, C, dtype)
        if slot == 0:                       # combination not compiled
            assert got == 0
            continue
        nchunk = -(-T // C)
        chains = B * H
        if nchunk == 0:
            assert got == 0
        elif chains * nchunk * slot <= cap:
            assert got == chains * nchunk * slot
        else:
            state = chains * dk * dv * 4
            assert got <= max(cap, 2 * chains * slot) + state
            assert got >= 2 * chains * slot + state
