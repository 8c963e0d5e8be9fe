"""The debug flag (SHAMPOO4_FLAG_DEBUG): every descriptor checked against the state and
workspace bounds at init, every workspace temporary filled with NaN before each call.

If any kernel read a temporary before writing it within a call (a value left over from
an earlier call, or never written), the NaN would reach the preconditioned gradient or
the state.  The kernels are deterministic, so with the flag every output and every state
byte must equal, bit for bit, those of the same steps without it; and the non-finite flag
stays clear.  Covered: the small-batch fused QR (one call per step, cached roots beside
the chain), ragged blocks through the three calls, the blocked QR of a large batch (its
products on the three-piece bf16 kernel), the float64 statistics update, the 32-bit
state, and a block with one diagonal side.
"""

import numpy as np
import pytest
import torch

from tests.gpu_util import announce, require_gpu, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    ("fused qr, one call", [(64, 32)], dict(bjorck_iters=1, root_cache=True), 1, True, None),
    ("ragged, three calls", [(40, 72), (130, 65), (1, 3)], dict(bjorck_iters=2), 2, False, None),
    ("blocked qr, x3 products", [(2048, 2048)], dict(bjorck_iters=1, root_cache=True), 1, True, None),
    ("float64 update", [(96, 40)], dict(bjorck_iters=1, root_cache=True, fp64_refresh=True), 2, True, None),
    ("32-bit state", [(70, 33), (16, 16)], dict(bjorck_iters=1, fp32_state=True), 1, False, None),
    ("diagonal side", [(48, 300)], dict(bjorck_iters=1, root_cache=True), 1, True, [(False, True)]),
]


def _run(shapes, cfg_kw, T, use_step, diagonal, debug, grads):
    from bit_quantized_shampoo_amd import Shampoo4Blocks, Shampoo4Config
    blocks = Shampoo4Blocks(shapes, Shampoo4Config(debug=debug, **cfg_kw), diagonal=diagonal)
    Ps = []
    for t, Gs in enumerate(grads, start=1):
        Gd = [to_dev(G) for G in Gs]
        if use_step:
            P = blocks.step(Gd, t, T)
        else:
            blocks.update_stats(Gd)
            if t % T == 0:
                blocks.refresh_root()
            P = blocks.precondition(Gd)
        torch.cuda.synchronize()
        Ps.append([p.cpu().numpy().copy() for p in P])
    assert blocks.check() == 0
    # each side's state buffers (the padding between them is never written)
    state = [blocks.side_state(b, side) for b in range(len(shapes)) for side in (0, 1)]
    blocks.close()
    return Ps, state


@pytest.mark.parametrize("label,shapes,cfg_kw,T,use_step,diagonal", CASES, ids=[c[0] for c in CASES])
def test_debug_flag_changes_nothing(label, shapes, cfg_kw, T, use_step, diagonal):
    require_gpu()
    rng = np.random.default_rng(11)
    steps = 3
    grads = [[(rng.standard_normal((m, n)) * 10.0 ** rng.uniform(-1, 1, size=(m, 1))).astype(np.float32)
              for (m, n) in shapes] for _ in range(steps)]
    announce(f"debug flag {label}: plain run")
    P0, s0 = _run(shapes, cfg_kw, T, use_step, diagonal, False, grads)
    announce(f"debug flag {label}: debug run")
    P1, s1 = _run(shapes, cfg_kw, T, use_step, diagonal, True, grads)
    for t in range(steps):
        for b in range(len(shapes)):
            assert np.all(np.isfinite(P1[t][b])), (label, t, b)
            assert np.array_equal(P0[t][b].view(np.uint32), P1[t][b].view(np.uint32)), (label, t, b)
    for a, b in zip(s0, s1):
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (label, k)
