"""GPU parity of the attention sublayer (GQA with RoPE) against the CPU oracle.

The core (moe_gqa_attention) is compared with oracle.gqa_attention_ref on the
same bf16 heads; the whole sublayer (moe_attention_block_forward) with
oracle.attention_sublayer_ref on the same bf16 activations and weights."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_wave_amd as moe
from synth import attention_heads, attention_inputs

from gpu_helpers import BF16_TOL, say, to_dev, to_host, widen_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()


@pytest.mark.parametrize("T,H,G", [
    (1, 4, 2), (2, 8, 8), (64, 4, 1), (100, 8, 2), (129, 4, 4), (300, 8, 1), (1000, 32, 8), (2048, 8, 2),
    # heads dealt to the 8 XCDs in runs of H/8: groups of 4 heads over 2 XCDs, groups of 8 over 3
    (700, 16, 4), (384, 24, 3),
])
def test_gqa_attention_core(T, H, G):
    say(f"gqa core T={T} H={H} G={G}")
    inp = attention_heads(T, H, G, 128, cfg_id=41 + T)
    o = moe.moe_gqa_attention(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]))
    torch.cuda.synchronize()
    ref = oracle.gqa_attention_ref(inp["q"], inp["k"], inp["v"], causal=True)
    got = widen_host(to_host(o))
    err = np.max(np.abs(got - ref))
    assert err <= BF16_TOL * np.max(np.abs(ref)), err
    # the first query attends to key 0 alone: its output is V[0] of its group, rounded once
    r = H // G
    v0 = widen_host(inp["v"][0])
    assert np.array_equal(got[0], np.repeat(v0, r, axis=0))


def test_gqa_attention_mixtral_t4096_sampled():
    """The benchmarked core: T = 4096, 32 query heads, 8 K/V groups, d_h = 128,
    the heads bench.py times (attention_heads, default seed), one launch as
    bench.py makes it.  Sampled queries (both sides of query-tile and key-tile
    boundaries, the last query, random ones) against the oracle one query at a
    time: query t is the last of t + 1 positions and sees keys 0..t."""
    T, H, G = 4096, 32, 8
    say(f"gqa core sampled T={T} H={H} G={G}")
    inp = attention_heads(T, H, G, 128)
    o = moe.moe_gqa_attention(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]))
    torch.cuda.synchronize()
    got = widen_host(to_host(o))
    rng = np.random.default_rng(11)
    ts = sorted({0, 1, 31, 32, 63, 64, 255, 256, 257, 2047, 2048, 3839, 3840, 4094, 4095,
                 *rng.integers(0, T, 17).tolist()})
    refs = [oracle.gqa_attention_ref(inp["q"][t:t + 1], inp["k"][:t + 1], inp["v"][:t + 1], causal=True)[0]
            for t in ts]
    scale = max(float(np.max(np.abs(r))) for r in refs)
    for t, ref in zip(ts, refs):
        err = float(np.max(np.abs(got[t] - ref)))
        assert err <= BF16_TOL * scale, (t, err)


def test_gqa_attention_is_deterministic_and_causal():
    say("gqa determinism / causality")
    T, H, G = 500, 8, 2
    inp = attention_heads(T, H, G, 128, cfg_id=77)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    a = moe.moe_gqa_attention(q, k, v).clone()
    b = moe.moe_gqa_attention(q, k, v).clone()
    k2, v2 = k.clone(), v.clone()
    k2[300:] = 0
    v2[300:] = 1
    c = moe.moe_gqa_attention(q, k2, v2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a[:300], c[:300]) and not torch.equal(a[300:], c[300:])


def _sublayer_case(T, d, H, G, pos0, theta, gamma, cfg_id=None):
    say(f"attention sublayer T={T} d={d} H={H} G={G} pos0={pos0} theta={theta} gamma={gamma}")
    inp = attention_inputs(T, d, H, G, 128, cfg_id=50 + T % 7 if cfg_id is None else cfg_id, gamma=gamma)
    h = to_dev(inp["h"])
    moe.moe_attention_block_forward(h, to_dev(inp["gamma"]), 1e-5, to_dev(inp["wqkv"]), to_dev(inp["wo"]), H, G,
                                    rope_theta=theta, pos0=pos0)
    torch.cuda.synchronize()
    nq, nkv = H * 128, G * 128
    wq, wk, wv = np.split(inp["wqkv"], [nq, nq + nkv])
    ref, *_ = oracle.attention_sublayer_ref(inp["h"], inp["gamma"], 1e-5, wq, wk, wv, inp["wo"], H, G, theta,
                                            pos0=pos0)
    got = widen_host(to_host(h))
    y_ref = ref - widen_host(inp["h"])
    tol = BF16_TOL * np.max(np.abs(y_ref)) + 2 ** -8 * np.max(np.abs(ref))
    err = np.max(np.abs(got - ref))
    assert err <= tol, (err, tol)


@pytest.mark.parametrize("T,d,H,G,pos0,theta,gamma", [
    (1, 512, 4, 2, 0, 1e6, "ones"),
    (37, 256, 2, 1, 5, 1e4, "random"),
    (200, 512, 4, 2, 0, 1e6, "random"),
    (300, 1024, 8, 2, 1000, 1e6, "ones"),
    (64, 512, 4, 4, 30000, 1e6, "random"),
    (65, 512, 4, 4, 30000, 1e6, "random"),  # the same one token past the streaming limit: fused epilogues
    (150, 256, 3, 1, 7, 1e4, "random"),  # Q|K|V width 640: a half-used last column tile
    (130, 512, 4, 2, 100000, 1e6, "random"),  # far positions through the GEMM epilogue's angle table
])
def test_attention_sublayer(T, d, H, G, pos0, theta, gamma):
    _sublayer_case(T, d, H, G, pos0, theta, gamma)


def test_attention_sublayer_mixtral_width():
    """Mixtral 8x7B widths (d = 4096, 32 query heads, 8 K/V groups, d_h = 128),
    1024 tokens: every output element against the oracle."""
    _sublayer_case(1024, 4096, 32, 8, 0, 1e6, "ones")


def test_attention_sublayer_mixtral_t4096():
    """The benchmarked sublayer: T = 4096 at Mixtral 8x7B widths (d = 4096,
    32 query heads, 8 K/V groups, theta = 1e6) on the inputs bench.py times
    (attention_inputs with its default seed): every output element against
    the oracle."""
    _sublayer_case(4096, 4096, 32, 8, 0, 1e6, "ones", cfg_id=40)
