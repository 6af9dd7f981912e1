"""GPU parity of the router load-balancing loss (moe_aux_loss) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_wave_amd as moe

from gpu_helpers import say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()


def _run(logits, k, alpha, mask):
    loss, stats = moe.moe_aux_loss(to_dev(logits), k=k, alpha=alpha,
                                   token_mask=None if mask is None else to_dev(mask.astype(np.uint8)),
                                   want_stats=True)
    torch.cuda.synchronize()
    return float(to_host(loss)[0]), to_host(stats)


@pytest.mark.parametrize("L,T,E,k,masked", [
    (3, 1000, 8, 2, True), (1, 4096, 8, 2, False), (2, 333, 16, 4, True), (1, 257, 64, 1, False),
    (4, 100, 2, 2, False), (32, 64, 8, 2, True),
])
def test_aux_loss_matches_oracle(L, T, E, k, masked):
    say(f"aux loss L={L} T={T} E={E} k={k} masked={masked}")
    rng = np.random.default_rng(L * 1000 + T + E)
    logits = (rng.standard_normal((L, T, E)) * 1.5).astype(np.float32)
    mask = (rng.uniform(size=T) > 0.25) if masked else None
    alpha = 0.01
    loss, stats = _run(logits, k, alpha, mask)
    f_ref, P_ref = oracle.router_stats_ref(list(logits), E, k, mask)
    ref = oracle.aux_loss_ref(list(logits), E, k, alpha, mask)
    f, P = stats[:k * E].reshape(k, E), stats[k * E:]
    np.testing.assert_allclose(f, f_ref, atol=1e-7)  # counts / N: exact up to one rounding
    np.testing.assert_allclose(P, P_ref, rtol=1e-5, atol=1e-7)
    assert abs(loss - ref) <= 1e-5 * abs(ref)


def test_aux_loss_uniform_load_is_alpha_k():
    say("aux loss uniform load")
    E, k, alpha = 8, 2, 0.01
    v = np.array([3.0, 2.0, 0.5, 0.1, -0.2, -1.0, -1.5, -2.0], np.float32)
    g = np.stack([np.roll(v, s) for s in range(E)] * 16)[None]  # every expert at every rank equally often
    loss, stats = _run(g, k, alpha, None)
    assert abs(loss - alpha * k) <= 1e-6


def test_aux_loss_no_valid_tokens_is_zero_and_deterministic():
    say("aux loss empty mask / determinism")
    rng = np.random.default_rng(3)
    g = rng.standard_normal((2, 500, 8)).astype(np.float32)
    loss, _ = _run(g, 2, 1.0, np.zeros(500, bool))
    assert loss == 0.0
    a, sa = _run(g, 2, 1.0, None)
    b, sb = _run(g, 2, 1.0, None)
    assert a == b and np.array_equal(sa, sb)


def test_aux_loss_from_router_logits_output():
    """The loss over the logits moe_route returns equals the oracle's loss over
    the oracle's own logits (routing-level agreement end to end)."""
    say("aux loss from moe_route logits")
    from synth import CONFIGS, generate
    cfg = CONFIGS["tiny_fp32"].with_(name="auxroute", cfg_id=12, T=512, d=256, d_ff=64, dtype="bf16")
    inp = generate(cfg, tensors=("x", "w_gate"))
    _, _, logits = moe.moe_route(to_dev(inp["x"]), to_dev(inp["w_gate"]), None, want_logits=True)
    loss, _ = moe.moe_aux_loss(logits, k=2, alpha=1.0)
    torch.cuda.synchronize()
    g_ref = oracle.router_logits(inp["x"], inp["w_gate"])
    ref = oracle.aux_loss_ref([g_ref], 8, 2, 1.0)
    assert abs(float(to_host(loss)[0]) - ref) <= 1e-3 * ref
