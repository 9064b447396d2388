"""pq2_gemv_tiles_static (the entry point that allocates nothing: its scratch
is a static device array of the library) against pq2_gemv_tiles with caller
scratch, through the C ABI: the same bits on calls in a row, each later one
smaller than the one before, so a stale array cannot pass for a fresh one;
the two-launch path (which uses the scratch) and the fused one (m <= 2,
k <= 8192) both taken; and the oracle's bound on the first case."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run_case(pq2, m, n, k, seed):
    print(f"[gpu-case] gemv static m={m} n={n} k={k}", flush=True)
    raw = workloads.make_raw_weights(n, k, seed=seed, codes="ternary+3", row_pad=2)
    x = workloads.make_activations(m, k, seed + 1, "normal+outliers")
    tiles = torch.empty(pq2.pq2_tiles_bytes(n, k), dtype=torch.uint8, device=DEV)
    pq2.pq2_prepare_tiles(torch.from_numpy(raw).to(DEV), n, k, tiles)
    xd = x.to(DEV)
    y_ref = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    qw = torch.empty((m, k), dtype=torch.int8, device=DEV)
    xw = torch.empty((m, k // 128), dtype=torch.float32, device=DEV)
    pq2.pq2_gemv_tiles(xd, tiles, y_ref, qw, xw)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    pq2.pq2_gemv_tiles_static(xd, tiles, y)
    torch.cuda.synchronize()
    a, b = y.cpu().numpy(), y_ref.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"static scratch differs at m={m} n={n} k={k}"
    return raw, x, a


def test_gemv_static_matches_caller_scratch():
    import gemm_int8_act_amd as pq2
    # Two-launch path (long k, then more than two columns), then the fused one.
    raw, x, y = _run_case(pq2, 4, 700, 17408, 501)
    qo, xso = oracle.quantize_act_i8(workloads.bf16_bits(x), "bf16")
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, 700, 17408)
    assert np.all(np.abs(y.astype(np.float64) - y_ref) <= bound)
    _run_case(pq2, 3, 300, 5120, 503)
    _run_case(pq2, 1, 200, 1024, 505)
