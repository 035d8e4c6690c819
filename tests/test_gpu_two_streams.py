"""The benchmark's two-stream layer step (the shared expert's FFN on a second
stream, as launches of its own: one group of T rows through offset views of
the h and Y buffers, 128-row tiles) against the one-stream step that the
layer parity tests check against the oracle: h', the h codes and scales, Y
and the expert counts must be identical bit for bit, since every GEMM row is
computed by the same per-slice arithmetic whatever launch or tile holds it."""
import pytest
import torch

import bench
import workloads
from helpers import say


RAGGED = workloads.custom_shape(T=37, d=640, E=12, K=4, I=384, outliers=True, name="custom")


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["tiny", "decode", "ragged"])
def test_two_stream_step_equals_one_stream_step(name):
    """ragged: 37 tokens, 12 experts top-4, d = 640, I = 384 (the shared
    expert's rows start at GEMM row 148, its h-scale view 148 * 3 floats into
    the buffer: 16-byte aligned, which the library requires)."""
    sh = RAGGED if name == "ragged" else workloads.SHAPES[name]
    assert bench.shared_views_aligned(sh)
    say(f"two-stream step, {name}: T={sh.T} E={sh.E} K={sh.K}")
    st = bench.layer_setup(sh)
    bench.layer_step(sh, st)
    torch.cuda.synchronize()
    ref = {k: st[k].clone() for k in ("out", "hq", "hs", "y")}
    ref_count = st["count"].clone()
    for k in ("out", "hq", "hs", "y"):
        st[k].fill_(7)                    # stale values must not survive
    for rep in range(2):                  # twice: nothing carries over from one step to the next
        bench.layer_step_two_streams(sh, st)
        torch.cuda.synchronize()
        for k in ("out", "hq", "y"):
            assert torch.equal(st[k], ref[k]), f"{k} differs (rep {rep})"
        assert torch.equal(st["hs"].view(torch.int32), ref["hs"].view(torch.int32)), f"hs differs (rep {rep})"
        assert torch.equal(st["count"], ref_count)
    # the bias update ran on the restored bias in both steps
    b1 = st["b_next"].clone()
    bench.layer_step(sh, st)
    torch.cuda.synchronize()
    assert torch.equal(st["b_next"], b1)


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_quant_beside_router_step_equals_one_stream_step(name):
    """The prefill benchmark's step: quant(u) and the bias restore copy on a
    second stream beside the router and dispatch; h', h, Y and the updated
    bias identical to the one-stream step's, over two steps in a row."""
    sh = RAGGED if name == "ragged" else workloads.SHAPES[name]
    say(f"quant beside the router, {name}: T={sh.T} E={sh.E} K={sh.K}")
    st = bench.layer_setup(sh)
    bench.layer_step(sh, st)
    torch.cuda.synchronize()
    ref = {k: st[k].clone() for k in ("out", "hq", "y", "b_next")}
    for k in ("out", "hq", "y", "b_next", "uq"):
        st[k].fill_(7)
    for rep in range(2):
        bench.layer_step_gemm_events(sh, st, bench.Events(), quant_beside_router=True)
        torch.cuda.synchronize()
        for k in ("out", "hq", "y", "b_next"):
            assert torch.equal(st[k], ref[k]), f"{k} differs (rep {rep})"
