"""GPU parity of mxq_attention_fp8 against the CPU oracle's block-scaled FP8 attention.

The probabilities' E4M3 codes are decisions taken from floating-point scores:
the kernel forms each score in the MFMA's fp32 accumulator, the oracle in
fp64.  Where an unquantized p * 2^8 lies within the fp32 accumulation bound
(D * 2^-24 of sum_d |q_d k_d|, for the score and the row's maximum)
of an E4M3 midpoint, both neighbours are correct codes; the oracle's
p_code_slack bounds what the other choice changes in each output (about 0.3 %
of the keys are such keys on these inputs).

Gate: the GEMM tolerance, normwise beyond the output's own bf16 rounding and
that slack, max((|y - r| - slack - halfulp(y))+) / max|r| <= 2e-3.  Leaving P
unquantized misses it by ~5x, unquantized attention by more; every case checks
the former.
"""

import numpy as np
import pytest

import oracle
from oracle import attention as att
from microscaling_quantized_diffusion_amd.inputs import bf16_bits_from_f32
from tests._util import bf16_out_to_f64, gpu_or_skip, log_case

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module")
def dev():
    return gpu_or_skip()


def _inputs(B, H, S, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    shape = (B, H, S, 128)
    q = bf16_bits_from_f32((rng.standard_normal(shape) * spread).astype(np.float32).reshape(-1, 128)).reshape(shape)
    k = bf16_bits_from_f32((rng.standard_normal(shape) * spread).astype(np.float32).reshape(-1, 128)).reshape(shape)
    v = bf16_bits_from_f32(rng.standard_normal(shape).astype(np.float32).reshape(-1, 128)).reshape(shape)
    return q, k, v


def _run(q, k, v, dev):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    t = [torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev) for x in (q, k, v)]
    out = mxq.attention_fp8(*t)
    torch.cuda.synchronize()
    return out


ETA = 128 * 2.0 ** -24  # fp32 accumulation bound over the 128 products of a score


def _gate(y, r, slack):
    return float(np.max(np.maximum(np.abs(y - r) - slack - oracle.bf16_half_ulp(y), 0.0)) / np.max(np.abs(r)))


def _check_head(out_head, q, k, v, rows=None):
    tq = att.quantize_qkv(q, k, v)
    qd = tq["q"] if rows is None else tq["q"][np.asarray(rows)]
    r = att.attend(qd, tq["k"], tq["v"])
    slack, _ = att.p_code_slack(qd, tq["k"], tq["v"], ETA)
    amb = len(att.near_midpoint_keys(qd, tq["k"], ETA))
    y = bf16_out_to_f64(out_head)
    err = _gate(y, r, slack)
    err_unq = _gate(y, att.attend(qd, tq["k"], tq["v"], quantize_probs=False), slack)
    print(f"attention error {err:.3e} (vs P unquantized {err_unq:.3e}), ambiguous P codes {amb} of "
          f"{qd.shape[0] * tq['k'].shape[0]}", flush=True)
    assert amb <= 0.01 * qd.shape[0] * tq["k"].shape[0]
    assert err <= TOL, err
    assert err_unq > TOL, err_unq


@pytest.mark.parametrize("B,H,S", [(1, 2, 256), (1, 1, 64), (1, 2, 320), (2, 3, 192)])
def test_attention_matches_oracle(B, H, S, dev):
    """Every output of every head; S = 64 and 320 leave the last 128-query tile partly empty."""
    log_case("attention", B, H, S)
    q, k, v = _inputs(B, H, S, seed=S + 7 * H)
    out = _run(q, k, v, dev).cpu()
    for b in range(B):
        for h in range(H):
            _check_head(out[b, h], q[b, h], k[b, h], v[b, h])


def test_attention_peaked_scores(dev):
    """Larger Q and K make each query attend to a few keys (max-dominated rows)."""
    log_case("attention peaked")
    q, k, v = _inputs(1, 2, 256, seed=3, spread=3.0)
    out = _run(q, k, v, dev).cpu()
    for h in range(2):
        _check_head(out[0, h], q[0, h], k[0, h], v[0, h])


def test_attention_max_in_last_key_tile(dev):
    """Every query's largest score is on the last key (channel 0 of Q is 3 and of that key 24), which sits
    in the last, half-filled 128-key tile of the maximum pass at S = 320: the P codes of all earlier keys
    are taken relative to it."""
    log_case("attention max in last tile")
    q, k, v = _inputs(1, 2, 320, seed=13)
    q, k = q.copy(), k.copy()
    q[..., 0] = bf16_bits_from_f32(np.full((1,), 3.0, dtype=np.float32))[0]
    k[..., -1, 0] = bf16_bits_from_f32(np.full((1,), 24.0, dtype=np.float32))[0]
    out = _run(q, k, v, dev).cpu()
    for h in range(2):
        _check_head(out[0, h], q[0, h], k[0, h], v[0, h])


def test_attention_deterministic(dev):
    import torch

    log_case("attention deterministic")
    q, k, v = _inputs(1, 4, 512, seed=5)
    a = _run(q, k, v, dev)
    b = _run(q, k, v, dev)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_attention_full_size_flux(dev):
    """FLUX-dev at 1024 x 1024: 24 heads, 4608 tokens (4096 image + 512 text), head dimension 128.
    Sampled query rows (the first and last included) of the first, a middle and the last head."""
    B, H, S = 1, 24, 4608
    log_case("attention full size", B, H, S)
    q, k, v = _inputs(B, H, S, seed=11)
    out = _run(q, k, v, dev)
    rng = np.random.default_rng(12)
    rows = np.union1d(rng.choice(S, 30, replace=False), [0, 127, 128, S - 1])
    import torch

    ri = torch.from_numpy(rows).to(out.device)
    for h in (0, 13, H - 1):
        _check_head(out[0, h][ri].cpu(), q[0, h], k[0, h], v[0, h], rows=rows)
