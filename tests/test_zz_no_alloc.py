"""The allocation-free grouped forward (bitlinear_forward_grouped_noalloc) against the
grouped forward with a caller workspace (bitlinear_forward_grouped_ws), through the C ABI.

Both run the same kernels; the no-alloc call takes its split-K partial products from the
library's static device array. Two calls in a row, the second with a smaller input, on
shapes that split K, must give the accumulators and outputs of the workspace call bit for
bit (and the oracle's accumulators on sampled rows)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
from test_parity_gpu import dev, host, random_product_inputs  # noqa: E402

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import ternary_quantized_linear_amd as m
    return m


def _entries(T, shapes, seed):
    ins, entries = [], []
    for i, (N, K) in enumerate(shapes):
        Xq, P, xs, beta = random_product_inputs(T, N, K, seed + i)
        ins.append((Xq, P, xs, beta))
        entries.append((dev(Xq), dev(xs), dev(P), dev(np.array([beta], np.float32)),
                        torch.empty((T, N), dtype=torch.float32, device="cuda:0"),
                        torch.empty((T, N), dtype=torch.int32, device="cuda:0")))
    return ins, entries


def _outputs(entries):
    return [(host(e[4]).copy(), host(e[5]).copy()) for e in entries]


def _run_both(bl, T, shapes, seed):
    ins, entries = _entries(T, shapes, seed)
    for (N, K) in shapes:
        assert bl.bitlinear_forward_choice(T, N, K) == "prefill"
        assert 0 < bl.bitlinear_forward_workspace_bytes(T, N, K) <= bl.NOALLOC_SCRATCH_BYTES
    nb = max(bl.bitlinear_forward_workspace_bytes(T, N, K) for (N, K) in shapes)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    print("no-alloc case: T=%d shapes=%s workspace=%d" % (T, shapes, nb), flush=True)
    bl.bitlinear_forward_grouped_ws(entries, T, ws)
    ref = _outputs(entries)
    for e in entries:            # poison the outputs, so a skipped store shows
        e[4].fill_(float("nan"))
        e[5].fill_(-1)
    bl.bitlinear_forward_grouped_noalloc(entries, T)
    got = _outputs(entries)
    for (Yr, ar), (Yg, ag), (Xq, P, xs, beta), (N, K) in zip(ref, got, ins, shapes):
        assert np.array_equal(ag, ar), "T=%d N=%d K=%d: accumulators differ" % (T, N, K)
        assert np.array_equal(Yg.view(np.uint32), Yr.view(np.uint32)), \
            "T=%d N=%d K=%d: outputs differ" % (T, N, K)
        rows = np.random.default_rng(N + K).choice(N, 24, replace=False)
        acc_o = oracle.product(Xq, P[rows], K)
        assert np.array_equal(ag[:, rows], acc_o), "T=%d N=%d K=%d: oracle rows" % (T, N, K)


def test_noalloc_matches_workspace_call_twice(bl):
    # first call: the 70B down shape and a 4096 x 16384 matrix at 64 tokens (K cut into
    # 8 and 16 slices); second call, smaller: the 4096 x 16384 matrix alone at 32 tokens
    _run_both(bl, 64, [(8192, 28672), (4096, 16384)], 1)
    _run_both(bl, 32, [(4096, 16384)], 2)
