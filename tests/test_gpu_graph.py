"""One layer step (forward, data backward, weight backward) captured in a HIP
graph through the C ABI and replayed: the library allocates nothing and
launches only kernels on the caller's stream, so the captured step must give
exactly the eager results.  Each replay runs on new inputs copied into the
captured buffers, with eager library calls and synchronisations between the
replays, and is compared bit for bit with an eager step on the same inputs
(the kernels are deterministic), and once against the oracle."""
import sys

import numpy as np
import pytest
import torch

import level_haar_wavelet_amd as wt
from level_haar_wavelet_amd import _native
from level_haar_wavelet_amd.synthetic import make_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests.gpu_util import DevInputs, assert_close, assert_grad_close

CASES = [
    # n, c, h, w, k, L, dtype: whole-plane kernels; a large plane (low-pass
    # pass, nested calls without the base path, tiled kernels); sides that 2^L
    # does not divide (padded copies)
    (4, 8, 56, 56, 5, 3, "f32"),
    (2, 4, 128, 128, 5, 3, "f16"),
    (2, 3, 30, 22, 3, 2, "f32"),
]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_captured_step_replays_match_eager(orc, case):
    n, c, h, w, k, L, dt = case
    _log("graph case %s" % (case,))
    code = 0 if dt == "f32" else 1
    tdt = torch.float32 if dt == "f32" else torch.float16
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=500 + h)
    d = DevInputs(inp, dt)
    y, dx = torch.empty_like(d.x), torch.empty_like(d.dy)
    grads = tuple(torch.empty_like(t) for t in (d.w_base, d.bias, d.s_base, d.w_lvl, d.s_lvl))
    ws = [torch.empty(max(wt.wtconv_workspace_size((n, c, h, w), k, L, code, op), 1), dtype=torch.uint8,
                      device="cuda") for op in (_native.OP_FWD, _native.OP_BWD_DATA, _native.OP_BWD_WEIGHT)]

    def step(s):
        wt.wtconv_forward(d.x, d.w_base, d.bias, d.s_base, d.w_lvl, d.s_lvl, y=y, stream=s, workspace=ws[0])
        wt.wtconv_backward_data(d.dy, d.w_base, d.s_base, d.w_lvl, d.s_lvl, dx=dx, stream=s, workspace=ws[1])
        wt.wtconv_backward_weight(d.x, d.dy, d.w_base, d.bias, d.s_base, d.w_lvl, d.s_lvl, workspace=ws[2],
                                  grads=grads, stream=s)

    def results():
        return [t.clone() for t in (y, dx) + grads]

    # warm the launch plans on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()

    cur = torch.cuda.current_stream()
    for r in range(3):
        new = make_inputs(n, c, h, w, k, L, dtype=dt, seed=900 + 7 * r)
        d.x.copy_(torch.from_numpy(new.x).to("cuda", dtype=tdt))
        d.dy.copy_(torch.from_numpy(new.dy).to("cuda", dtype=tdt))
        # outputs poisoned, so a replay that skips a kernel shows
        for t in (y, dx) + grads:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = results()
        step(cur)  # eager on the same inputs
        torch.cuda.synchronize()
        ref = results()
        for a, b, name in zip(got, ref, ("y", "dx", "dw_base", "dbias", "ds_base", "dw_lvl", "ds_lvl")):
            assert torch.equal(a, b), "replay %d: %s differs from the eager step" % (r, name)
        if r == 0:
            xo = new.x.astype(np.float64)
            dyo = new.dy.astype(np.float64)
            # the parameters stay those captured with (inp's)
            assert_close(got[0], orc.forward(xo, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L), dt,
                         "graph y")
            assert_close(got[1], orc.backward_data(dyo, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L), dt,
                         "graph dx")
            refg = orc.backward_weight(xo, dyo, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
            for gg, rr, name in zip(got[2:], refg, ("dw_base", "dbias", "ds_base", "dw_lvl", "ds_lvl")):
                assert_grad_close(gg, rr, dt, "graph " + name)
