"""Shared helpers of the GPU parity tests: host/device marshalling and the
comparison rules (routing by logit gap, weights keyed by expert, outputs
relative to max|y_ref|)."""
import sys

import numpy as np
import torch

GAP = 1e-4          # routing compared bit-exactly only where g_(2) - g_(3) > GAP
W_TOL = 1e-6        # combine weights, absolute
BF16_TOL = 2e-2     # outputs, relative to max|y_ref|, bf16 experts
F32_TOL = 1e-4      # outputs, relative to max|y_ref|, fp32 experts


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_host(t):
    """GPU tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def widen_host(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return a.astype(np.float32)


def clear_tokens(g_ref, gap=GAP):
    s = np.sort(g_ref.astype(np.float64), axis=1)[:, ::-1]
    if s.shape[1] == 2:  # k == E: every expert is selected, the set is never in doubt
        s = np.concatenate([s, np.full((s.shape[0], 1), -np.inf)], axis=1)
    clear = (s[:, 1] - s[:, 2]) > gap
    ordered = clear & ((s[:, 0] - s[:, 1]) > gap)
    return clear, ordered


def check_routing(g_ref, idx_ref, w_ref, idx_gpu, w_gpu, gap=GAP):
    """Top-2 sets equal on every clear token, slot order where slot 0 is clear,
    weights within W_TOL keyed by (token, expert).  Returns the clear mask."""
    clear, ordered = clear_tokens(g_ref, gap)
    T = g_ref.shape[0]
    for t in range(T):
        assert idx_gpu[t, 0] != idx_gpu[t, 1], f"token {t}: repeated expert"
        assert 0 <= idx_gpu[t].min() and idx_gpu[t].max() < g_ref.shape[1]
        np.testing.assert_allclose(w_gpu[t].sum(), 1.0, atol=1e-6)
    bad = [t for t in np.nonzero(clear)[0] if set(idx_gpu[t]) != set(idx_ref[t])]
    assert not bad, f"routing differs on clear tokens {bad[:10]}"
    bad = [t for t in np.nonzero(ordered)[0] if idx_gpu[t, 0] != idx_ref[t, 0]]
    assert not bad, f"slot order differs on tokens {bad[:10]}"
    for t in np.nonzero(clear)[0]:
        for s in range(2):
            j = int(np.nonzero(idx_ref[t] == idx_gpu[t, s])[0][0])
            assert abs(float(w_gpu[t, s]) - float(w_ref[t, j])) <= W_TOL, (t, s)
    return clear


def check_dispatch_on_clear(idx_gpu, off_gpu, st_gpu, inv_gpu, clear, E):
    """The GPU permutation is valid for its own indices, and per expert the token
    lists agree with the oracle's once near-tie tokens are removed."""
    T = idx_gpu.shape[0]
    assert off_gpu[0] == 0 and off_gpu[E] == 2 * T and np.all(np.diff(off_gpu) >= 0)
    for e in range(E):
        rows = st_gpu[off_gpu[e]:off_gpu[e + 1]]
        assert np.all(np.diff(rows) > 0), f"expert {e} rows not ascending"
        assert np.all(np.any(idx_gpu[rows] == e, axis=1))
    for t in range(T):
        for s in range(2):
            r = inv_gpu[t, s]
            assert st_gpu[r] == t and off_gpu[idx_gpu[t, s]] <= r < off_gpu[idx_gpu[t, s] + 1]


def max_rel_err(y, y_ref, mask=None):
    y = widen_host(y) if y.dtype == np.uint16 else y
    if mask is not None:
        y, y_ref = y[mask], y_ref[mask]
    scale = float(np.max(np.abs(y_ref)))
    return float(np.max(np.abs(y.astype(np.float64) - y_ref))) / max(scale, 1e-30)
