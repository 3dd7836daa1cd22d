"""kda_fwd_chunked_noalloc (the prefill with the library's own device array
in place of a workspace) against kda_fwd_chunked_ex on the same inputs,
through the C ABI: two calls in a row, the second with a smaller input, so
the array is reused with stale contents from the first."""
import numpy as np
import pytest

import oracle
from synth import prefill_inputs
from tests.gpu_harness import TOL, log, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


def _call(x, dtype, C, gate, rule, *, noalloc, want_state=True):
    import torch
    import gated_delta_rule_76_amd as kda
    q, k, v, a, b = (to_dev(x[n], dtype) for n in ("q", "k", "v", "alpha", "beta"))
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    s0 = torch.from_numpy(x["S0"]).cuda()
    o = torch.full((B, T, H, dv), float("nan"), dtype=q.dtype, device="cuda")
    st = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device="cuda") if want_state else None
    code = kda.KDA_BF16 if dtype == "bf16" else kda.KDA_F32
    g, r = kda.GATES[gate], kda.RULES[rule]
    stream = torch.cuda.current_stream().cuda_stream
    stp = st.data_ptr() if st is not None else None
    if noalloc:
        rc = kda.kda_fwd_chunked_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(),
                                             b.data_ptr(), s0.data_ptr(), o.data_ptr(), stp, B, T, H,
                                             dk, dv, C, code, g, r, stream)
    else:
        need = kda.workspace_bytes(B, T, H, dk, dv, C, code)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        rc = kda.kda_fwd_chunked_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(),
                                     b.data_ptr(), s0.data_ptr(), o.data_ptr(), stp, B, T, H, dk,
                                     dv, C, code, ws.data_ptr(), need, stream, g, r)
    assert rc == 0, kda.status_string(rc)
    torch.cuda.synchronize()
    return to_np(o), (to_np(st) if st is not None else None)


@pytest.mark.parametrize("dtype,dk,C,big,small,gate,rule", [
    # the first call needs many segments of the 64 MiB array, the second fits at once
    ("bf16", 128, 64, (4, 4096, 16), (1, 300, 3), "channel", "delta"),
    ("bf16", 128, 64, (1, 40000, 8), (2, 129, 5), "head", "linear"),
    ("f32", 128, 32, (2, 3000, 8), (1, 77, 2), "none", "delta"),
])
def test_noalloc_matches_workspace_path(dtype, dk, C, big, small, gate, rule):
    for i, (B, T, H) in enumerate((big, small)):
        log(f"[noalloc] call {i + 1}: {dtype} dk{dk} C{C} B{B} T{T} H{H} gate {gate} rule {rule}")
        x = prefill_inputs(B, T, H, dk, dk, dtype=dtype, gate_c=0.1, s0_std=0.05, seed=T + H)
        if gate == "head":
            x["alpha"] = np.ascontiguousarray(x["alpha"][..., 0])
        o1, s1 = _call(x, dtype, C, gate, rule, noalloc=False)
        o2, s2 = _call(x, dtype, C, gate, rule, noalloc=True)
        np.testing.assert_array_equal(o2, o1)
        np.testing.assert_array_equal(s2, s1)
        o3, s3 = _call(x, dtype, C, gate, rule, noalloc=True, want_state=False)
        assert s3 is None
        np.testing.assert_array_equal(o3, o1)
        if i == 1:   # the small call against the oracle as well
            o_ref, s_ref = oracle.kda_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                                              x["S0"], gate=gate, rule=rule)
            eo, es = rel_err(o2, o_ref), rel_err(s2, s_ref)
            log(f"[noalloc] small call rel_err o={eo:.3e} S_T={es:.3e}")
            assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_noalloc_rejects_sizes_beyond_the_array():
    import gated_delta_rule_76_amd as kda
    P = 0x100000   # never dereferenced: the size check fails before any launch
    rc = kda.kda_fwd_chunked_noalloc_raw(P, P, P, P, P, None, P, None, 400, 1 << 14, 1, 128, 128,
                                         64, kda.KDA_BF16)
    assert rc == 3   # KDA_ERR_WORKSPACE
