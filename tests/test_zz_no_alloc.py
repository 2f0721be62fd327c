"""rtp_decode_step_static (the decode step on the library's static device
scratch, for callers that cannot allocate) against rtp_decode_step with a
workspace: same kernels, so the outputs and selected sets are bit-identical.
Two calls in a row, the second on a smaller input, then a layer of another
layout (its persistent state is cleared), then the first again."""
import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import gen
import long_context_sparse_retrieval_amd as rtp
import oracle as O
from parity import dev_bf16, layer_of, say

pytestmark = pytest.mark.gpu


def _inputs(spec, seed):
    wl = gen.make_workload(spec, seed)
    kc, ki = O.build_caches(wl)
    return wl, [dev_bf16(x) for x in (wl.q_pre, wl.w_q, ki, kc, wl.v)]


def _both(lay, args):
    cap = lay.N
    outs = []
    for fn in ("ws", "static"):
        idx = torch.full((lay.B, lay.Hr, 1, cap), -1, dtype=torch.int32, device="cuda")
        cnt = torch.zeros((lay.B, lay.Hr, 1), dtype=torch.int32, device="cuda")
        if fn == "ws":
            out = rtp.decode_step(lay, *args, rtp.workspace(lay), idx=idx, count=cnt)
        else:
            out = rtp.decode_step_static(lay, *args, idx=idx, count=cnt)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()))
    return outs


def _same(a, b, what):
    assert np.array_equal(a[0], b[0]), f"{what}: outputs differ"
    assert np.array_equal(a[2], b[2]), f"{what}: counts differ"
    for bb in range(a[2].shape[0]):
        for r in range(a[2].shape[1]):
            c = int(a[2][bb, r, 0])
            assert np.array_equal(a[1][bb, r, 0, :c], b[1][bb, r, 0, :c]), f"{what}: sets differ b{bb} r{r}"


def test_static_step_matches_workspace_step():
    rtp.load()
    spec = gen.spec_for(3, B=2, N=20000, window=1024, query_scale="unit")
    say(f"static step, first call: {spec}")
    scales = {(b, r): 0.35 * (1.0 + 0.5 * ((b * spec.Hr + r) % 2)) for b in range(spec.B) for r in range(spec.Hr)}
    wl, args = _inputs(spec, 7)
    lay = layer_of(spec, rtp)
    assert rtp.workspace_bytes(lay) <= rtp.STATIC_SCRATCH_BYTES
    a, b = _both(lay, args)
    _same(a, b, "first call")
    # second call in a row, a smaller input on the same layer layout
    small = dataclasses.replace(lay, N=6000, Ncap=spec.N)
    say("static step, second call: N=6000 on the same caches")
    a2, b2 = _both(small, args)
    _same(a2, b2, "second call (smaller)")
    # another layout (batch 1, other heads), then the first layout again
    spec3 = gen.spec_for(2, B=1, N=3000, window=512)
    say(f"static step, other layout: {spec3}")
    wl3, args3 = _inputs(spec3, 9)
    a3, b3 = _both(layer_of(spec3, rtp), args3)
    _same(a3, b3, "other layout")
    a4, b4 = _both(lay, args)
    _same(a4, b4, "first layout again")
    assert np.array_equal(a4[0], a[0])


def test_static_step_rejects_layers_beyond_the_scratch():
    """Checked before any device work: the status, nothing launched."""
    lay = rtp.Layer(B=64, Hq=64, Hkv=8, N=1 << 20, head_mode=[1] * 64)
    assert rtp.workspace_bytes(lay) > rtp.STATIC_SCRATCH_BYTES
    q = torch.zeros((1,), dtype=torch.bfloat16, device="cuda")
    p = q.data_ptr()
    st = rtp.load().rtp_decode_step_static(ctypes.byref(lay.c()), p, p, p, p, p, p, None, None, 0, rtp._stream())
    assert st == -3
