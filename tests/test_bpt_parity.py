"""GPU parity of the blockwise attention + feed-forward layer (fa_bpt_layer) against the
fp64 oracle (bpt_layer_ref), through the C ABI.

Tolerance, derived from the path's roundings (the stated bar covers attention outputs
only): oracle.fullcheck.ffn_sigma gives the standard deviation of the rounding error of y
(h rounded to bf16 before the first product, the hidden activations after the ReLU);
per element |y' - y| <= 1e-2 + half a bf16 spacing of y + 6 sigma, and per tensor the
forward's rel-L2 bar plus 2 ||sigma|| / ||y|| (oracle.fullcheck.check_ffn). The
full-size layer is checked on every element.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import fullcheck as fc
from oracle.attention import attention_ref, ffn_ref, widen_bf16
from synth import WORKLOADS, make_ffn_weights, make_qkv, make_workload
from tests.parity import up

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_21_amd as fa
    return fa


def _sigma(h, w1, b1, w2):
    return fc.ffn_sigma(h, w1, b1, w2)


def _check(y_gpu, y, sigma, what="bpt"):
    err = np.abs(y_gpu - y)
    bound = fc.ffn_bound(y, sigma)
    idx = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.isfinite(y_gpu).all(), f"{what}: non-finite output"
    assert (err <= bound).all(), f"{what}: |err| {err[idx]:.4e} > bound {bound[idx]:.4e} at {idx}"
    ny = np.linalg.norm(y)
    rel = np.linalg.norm(y_gpu - y) / ny
    rel_bound = fc.REL_L2 + 2.0 * np.linalg.norm(sigma) / ny
    assert rel <= rel_bound, f"{what}: rel-L2 {rel:.3e} > {rel_bound:.3e}"
    return {"max_abs": float(err.max()), "max_err_over_bound": float((err / bound).max()), "rel_l2": float(rel),
            "rel_l2_bound": float(rel_bound)}


def _run(fa, q, k, v, w, causal, scale, block_rows):
    tw = [up(x) for x in w]
    y = fa.bpt_layer(up(q), up(k), up(v), *tw, causal=causal, scale=scale, block_rows=block_rows)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


SMALL = [
    # B, Hq, Hkv, S, d, block_rows
    (1, 2, 2, 100, 64, 64), (2, 2, 1, 130, 64, 32), (1, 4, 2, 257, 64, 100), (1, 2, 2, 200, 128, 200),
    (1, 1, 1, 1, 64, 16), (2, 2, 2, 96, 64, 1000),
    # 11 x 2 tiles in the first product: a ragged group of the grouped tile order
    (1, 2, 2, 2700, 64, 2700),
    # d_model 192 and 320: odd numbers of 64-wide k stages (3 and 5) in the first product
    (1, 3, 3, 150, 64, 64), (2, 5, 5, 70, 64, 70),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=[str(s) for s in SMALL])
def test_small_shapes(fa, shape, causal):
    B, Hq, Hkv, S, d, rows = shape
    print(f"case {shape} causal={causal}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, S, S, d, seed=900 + S + d)
    dm = Hq * d
    w = make_ffn_weights(dm, 4 * dm, seed=901 + dm)
    scale = 1.0 / math.sqrt(d)
    y_gpu = _run(fa, q, k, v, w, causal, scale, rows)
    W = [widen_bf16(x) for x in w]
    O = attention_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), causal=causal, scale=scale)[0]
    h = O.reshape(B * S, dm)
    y = ffn_ref(h, *W).reshape(B, S, dm)
    info = _check(y_gpu, y, _sigma(h, W[0], W[1], W[2]).reshape(B, S, dm))
    print("  ", info, flush=True)


def test_block_size_does_not_change_the_function(fa):
    q, k, v = make_qkv(1, 2, 2, 300, 300, 64, seed=95)
    w = make_ffn_weights(128, 512, seed=96)
    a = _run(fa, q, k, v, w, True, 0.125, 64)
    b = _run(fa, q, k, v, w, True, 0.125, 300)
    W = [widen_bf16(x) for x in w]
    O = attention_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), causal=True, scale=0.125)[0].reshape(300, 128)
    y = ffn_ref(O, *W).reshape(1, 300, 128)
    sig = _sigma(O, W[0], W[1], W[2]).reshape(1, 300, 128)
    for yy in (a, b):
        _check(yy, y, sig)


def test_full_size_long_prefill_every_element(fa):
    """Blockwise layer on the MHA long prefill (B2 H32 S8192 d128 causal, K x4 on 1% of
    positions) with d_model 4096 and d_ff 16384, 2048-row blocks (the benchmark's
    configuration): every element of y against the oracle (attention over the process
    pool, the feed-forward network in row blocks)."""
    wl = WORKLOADS["mha8k"]
    q, k, v = make_workload(wl)
    dm = wl.Hq * wl.d
    w = make_ffn_weights(dm, 4 * dm, seed=wl.seed)
    print(f"full-size blockwise layer {wl.name}, d_ff {4 * dm}", flush=True)
    y_gpu = _run(fa, q, k, v, w, True, wl.scale, 2048).reshape(wl.B * wl.Sq, dm)
    O = fc.attention_outputs(q, k, v, causal=True, scale=wl.scale, progress=lambda m: print("  ", m, flush=True))
    res = fc.check_ffn(O.reshape(wl.B * wl.Sq, dm), w, y_gpu, progress=lambda m: print("  ", m, flush=True))
    print("  ", res, flush=True)
    path = os.environ.get("FA_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"workload": wl.name, "layer": "blockwise attention + feed-forward, d_ff 16384, "
                                "2048-row blocks", "label": "pass" if fc.ffn_ok(res) else "fail", "y": res}) + "\n")
    assert fc.ffn_ok(res), res
