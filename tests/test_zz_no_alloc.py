"""spec_verify_static (the workspace in the library's static device array)
against spec_verify with a caller workspace, through the C ABI, on an MI355X:
the same outputs bit for bit on consecutive calls, each smaller than the one
before, so that a call finds the array holding the previous call's data; and
the call captured in a HIP graph (torch's graph capture on a side stream),
every replay -- with eager work and synchronisations between them -- giving
the eager call's outputs bit for bit: the library enqueues only kernels (no
memset, copy or allocation).  Every case prints its shape before touching
the GPU."""

import sys

import numpy as np
import pytest

from synth import inputs as I
from tests import parity

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


CASES = [  # (B, gamma, d, V, seed), largest first; R > 64 takes the tiled GEMM
    (16, 4, 512, 20000, 41),     # R = 80
    (4, 4, 256, 30000, 42),      # R = 20
    (2, 3, 128, 5000, 43),       # R = 8
]


def test_static_workspace_matches_spec_verify():
    import torch
    import draft_token_verification_02_amd as sv
    assert torch.cuda.is_available(), "no ROCm device"
    sv.library()
    dev = torch.device("cuda:0")
    for B, gamma, d, V, seed in CASES:
        _say(f"static workspace B={B} gamma={gamma} d={d} V={V} seed={seed}")
        x = I.custom(B, gamma, d, V, seed=seed, sigma=0.8, w_std=parity.small_w_std(d))
        t = parity.to_device(x, dev)
        ref_out, ref_n = sv.verify(t["hidden_bits"], t["W_bits"], t["draft"], t["q"],
                                   t["uniforms"])
        out = torch.full((B, gamma + 1), -7, dtype=torch.int32, device=dev)
        n = torch.full((B,), -7, dtype=torch.int32, device=dev)
        sv.verify_static(t["hidden_bits"], t["W_bits"], t["draft"], t["q"], t["uniforms"],
                         out_tokens=out, n_accepted=n)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), ref_out.cpu().numpy())
        np.testing.assert_array_equal(n.cpu().numpy(), ref_n.cpu().numpy())
        # and against the oracle, to the usual bar (outputs only: the static
        # workspace has no debug views)
        rep = parity.compare(x, {**parity.run_gpu(x, dev), "out": out.cpu().numpy(),
                                 "n": n.cpu().numpy()})
        _say(f"static workspace ok: n={n.cpu().tolist()} draws exact={rep['draw_exact']}")
        del t


def test_static_workspace_rejects_dims_beyond_its_size():
    import torch
    import draft_token_verification_02_amd as sv
    from draft_token_verification_02_amd import _lib
    dev = torch.device("cuda:0")
    B, gamma, d, V = 20, 4, 64, 128256         # 100 rows: 52.7 MB of workspace
    _say(f"static workspace too small B={B} gamma={gamma} d={d} V={V}")
    h = torch.zeros((B, gamma + 1, d), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((V, d), dtype=torch.bfloat16, device=dev)
    draft = torch.zeros((B, gamma), dtype=torch.int32, device=dev)
    q = torch.zeros((B, gamma, V), dtype=torch.float32, device=dev)
    u = torch.ones((B, gamma + 1), dtype=torch.float32, device=dev)
    with pytest.raises(sv.SVError, match="more than the static"):
        sv.verify_static(h, W, draft, q, u)
    assert _lib.workspace_bytes(_lib.Dims(B, gamma, d, V)) > _lib.STATIC_SCRATCH_BYTES


@pytest.mark.parametrize("B, gamma, d, V, seed, tiled", [(4, 4, 256, 30000, 51, False),
                                                         (16, 4, 512, 20000, 52, False),
                                                         (16, 4, 512, 20000, 53, True)])
def test_static_workspace_replays_in_a_graph(B, gamma, d, V, seed, tiled):
    import torch
    import draft_token_verification_02_amd as sv
    assert torch.cuda.is_available(), "no ROCm device"
    sv.library()
    dev = torch.device("cuda:0")
    _say(f"static workspace in a graph B={B} gamma={gamma} d={d} V={V} seed={seed} tiled W={tiled}")
    x = I.custom(B, gamma, d, V, seed=seed, sigma=0.8, w_std=parity.small_w_std(d))
    t = parity.to_device(x, dev)
    args = (t["hidden_bits"], parity.gpu_w(t, tiled), t["draft"], t["q"], t["uniforms"])
    ref_out, ref_n = sv.verify_static(*args)          # eager; also resolves the array's address
    torch.cuda.synchronize()
    ref_out, ref_n = ref_out.cpu().numpy(), ref_n.cpu().numpy()
    out = torch.full((B, gamma + 1), -7, dtype=torch.int32, device=dev)
    n = torch.full((B,), -7, dtype=torch.int32, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        sv.verify_static(*args, out_tokens=out, n_accepted=n)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(-7)                                 # eager work between the replays
        n.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), ref_out, err_msg=f"replay {rep}")
        np.testing.assert_array_equal(n.cpu().numpy(), ref_n, err_msg=f"replay {rep}")
    _say(f"graph replays ok: n={ref_n.tolist()}")
    del graph, t
