"""C ABI on the host: the library loads, exports every declared symbol, and
validates arguments before launching anything (no GPU needed)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest
import torch

from sparse_mixture_experts_wave_amd import _lib, moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

# A 16-byte aligned address that is never dereferenced: every call below
# fails validation (or returns for T == 0) before it could be used.
FAKE = ctypes.c_void_p(0x10000)
MISALIGNED = ctypes.c_void_p(0x10008)


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(moe_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward",
            "moe_block_forward", "moe_workspace_size", "moe_last_error", "moe_attention_workspace_size",
            "moe_gqa_attention", "moe_attention_block_forward"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def shape(T=16, d=4096, d_ff=14336, E=8, k=2, act=_lib.MOE_BF16, wt=None):
    return _lib.MoEShape(T, d, d_ff, E, k, act, act if wt is None else wt)


def route(lib, s, x=FAKE, wg=FAKE, idx=FAKE, w=FAKE):
    return lib.moe_route(ctypes.byref(s), x, wg, None, None, idx, w, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), _lib.MOE_ERR_INVALID_ARG),
    (dict(d=100), _lib.MOE_ERR_INVALID_ARG),
    (dict(d=0), _lib.MOE_ERR_INVALID_ARG),
    (dict(d_ff=96), _lib.MOE_ERR_INVALID_ARG),
    (dict(E=1), _lib.MOE_ERR_INVALID_ARG),
    (dict(E=65), _lib.MOE_ERR_INVALID_ARG),
    (dict(k=0), _lib.MOE_ERR_INVALID_ARG),
    (dict(k=9), _lib.MOE_ERR_INVALID_ARG),      # k outside 1..E: the pages' ValueError
    (dict(E=16, k=9), _lib.MOE_ERR_UNSUPPORTED),
    (dict(E=6), _lib.MOE_ERR_UNSUPPORTED),
    (dict(act=_lib.MOE_BF16, wt=_lib.MOE_F32), _lib.MOE_ERR_UNSUPPORTED),
    (dict(act=7), _lib.MOE_ERR_INVALID_ARG),
    (dict(T=1 << 25, d=64), _lib.MOE_ERR_UNSUPPORTED),  # T * d = 2^31: 32-bit activation offsets
])
def test_shape_validation(lib, kw, status):
    assert route(lib, shape(**kw)) == status
    assert lib.moe_last_error().decode() != ""


def test_null_and_misaligned_pointers(lib):
    s = shape()
    assert route(lib, s, x=None) == _lib.MOE_ERR_INVALID_ARG
    assert b"x is NULL" in lib.moe_last_error()
    assert route(lib, s, wg=MISALIGNED) == _lib.MOE_ERR_INVALID_ARG
    assert b"aligned" in lib.moe_last_error()
    assert lib.moe_route(ctypes.byref(s), FAKE, FAKE, MISALIGNED, None, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_route(None, FAKE, FAKE, None, None, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG


def test_zero_tokens_is_a_no_op(lib):
    s = shape(T=0)
    assert route(lib, s) == _lib.MOE_OK
    assert lib.moe_combine(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, None) == _lib.MOE_OK
    assert lib.moe_forward(ctypes.byref(s), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, ctypes.c_void_p(0x20000),
                           None, 0, None) == _lib.MOE_OK
    assert lib.moe_expert_ffn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 0,
                              None) == _lib.MOE_OK


GEMM_PARTIALS = 256 * 256 * 256 * 4  # split-K partial sums of the bf16 grouped GEMM (T > 64)


def test_workspace_sizes(lib):
    s = shape(T=4096)
    rows = 4096 * 2
    ws = lib.moe_workspace_size(ctypes.byref(s))
    # h (bf16) + y_sorted (fp32) + normalised input + GEMM partial sums dominate
    need = rows * 14336 * 2 + rows * 4096 * 4 + 4096 * 4096 * 2 + GEMM_PARTIALS
    assert need <= ws < need + (1 << 20)
    assert lib.moe_expert_ffn_workspace_size(ctypes.byref(s)) == rows * 14336 * 2 + GEMM_PARTIALS
    # the streaming path (T <= 64) needs no partial sums
    small = shape(T=64)
    assert lib.moe_expert_ffn_workspace_size(ctypes.byref(small)) == 64 * 2 * 14336 * 2
    assert lib.moe_workspace_size(ctypes.byref(shape(d=100))) == 0
    assert lib.moe_workspace_size(None) == 0


def test_workspace_too_small_is_rejected(lib):
    s = shape(T=16)
    st = lib.moe_forward(ctypes.byref(s), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, ctypes.c_void_p(0x20000),
                         FAKE, 1024, None)
    assert st == _lib.MOE_ERR_INVALID_ARG and b"workspace" in lib.moe_last_error()
    st = lib.moe_expert_ffn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 16, None)
    assert st == _lib.MOE_ERR_INVALID_ARG


def test_forward_rejects_aliased_output(lib):
    s = shape(T=16)
    st = lib.moe_forward(ctypes.byref(s), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 40, None)
    assert st == _lib.MOE_ERR_INVALID_ARG and b"alias" in lib.moe_last_error()


def test_noalloc_forward_host_checks(lib):
    """moe_forward_noalloc: its 64 MiB static buffer holds 744 Mixtral tokens'
    intermediates; 745 are refused before any device call, as are an aliased
    output and NULL weights.  T = 0 is a no-op."""
    y = ctypes.c_void_p(0x20000)
    st = lib.moe_forward_noalloc(ctypes.byref(shape(T=745)), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, y, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED and b"static scratch" in lib.moe_last_error()
    st = lib.moe_forward_noalloc(ctypes.byref(shape(T=16)), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, None)
    assert st == _lib.MOE_ERR_INVALID_ARG and b"alias" in lib.moe_last_error()
    st = lib.moe_forward_noalloc(ctypes.byref(shape(T=16)), FAKE, FAKE, None, None, FAKE, FAKE, None, y, None)
    assert st == _lib.MOE_ERR_INVALID_ARG and b"w1 is NULL" in lib.moe_last_error()
    assert lib.moe_forward_noalloc(ctypes.byref(shape(T=0)), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, y,
                                   None) == _lib.MOE_OK
    # the limit: 744 tokens' routing, permutation, h and y_sorted fit 64 MiB, 745 do not
    per = lambda T: sum(-(-n // 256) * 256 for n in (8 * T, 8 * T, 36, 8 * T, 8 * T, 2 * T * 14336 * 2,
                                                       2 * T * 4096 * 4))
    assert per(744) <= 64 << 20 < per(745)


def test_expert_bias_pointers_are_validated(lib):
    s = shape(T=16)
    bad = _lib.MoEExpertBias(None, MISALIGNED, None)
    st = lib.moe_forward(ctypes.byref(s), FAKE, FAKE, None, FAKE, FAKE, FAKE, ctypes.byref(bad),
                         ctypes.c_void_p(0x20000), FAKE, 1 << 40, None)
    assert st == _lib.MOE_ERR_INVALID_ARG and b"expert_bias->b3" in lib.moe_last_error()
    st = lib.moe_expert_ffn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(bad), FAKE, FAKE,
                            1 << 40, None)
    assert st == _lib.MOE_ERR_INVALID_ARG and b"expert_bias->b3" in lib.moe_last_error()
    st = lib.moe_block_forward(ctypes.byref(s), FAKE, FAKE, 1e-5, FAKE, None, FAKE, FAKE, FAKE, ctypes.byref(bad),
                               FAKE, 1 << 40, None)
    assert st == _lib.MOE_ERR_INVALID_ARG and b"expert_bias->b3" in lib.moe_last_error()


def test_block_forward_validates_eps(lib):
    s = shape(T=16)
    st = lib.moe_block_forward(ctypes.byref(s), FAKE, FAKE, 0.0, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                               None)
    assert st == _lib.MOE_ERR_INVALID_ARG and b"eps" in lib.moe_last_error()


def test_python_binding_maps_status_to_exceptions(lib):
    with pytest.raises(ValueError):
        _lib.check(route(lib, shape(d=100)))
    with pytest.raises(NotImplementedError):
        _lib.check(route(lib, shape(E=16, k=9)))
    _lib.check(_lib.MOE_OK)


# ---------------------------------------------------------------------------
# attention sublayer entry points (validation only: no GPU here)
# ---------------------------------------------------------------------------
def attn_shape(T=128, d=4096, H=32, G=8, d_h=128, act=_lib.MOE_BF16):
    return _lib.MoEAttnShape(T, d, H, G, d_h, act)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), _lib.MOE_ERR_INVALID_ARG),
    (dict(d=100), _lib.MOE_ERR_INVALID_ARG),
    (dict(H=32, G=6), _lib.MOE_ERR_INVALID_ARG),
    (dict(G=0), _lib.MOE_ERR_INVALID_ARG),
    (dict(d_h=127), _lib.MOE_ERR_INVALID_ARG),
    (dict(d_h=64), _lib.MOE_ERR_UNSUPPORTED),
    (dict(act=_lib.MOE_F32), _lib.MOE_ERR_UNSUPPORTED),
    (dict(act=9), _lib.MOE_ERR_INVALID_ARG),
    (dict(T=1 << 19), _lib.MOE_ERR_UNSUPPORTED),  # T * (H + 2G) * d_h >= 2^31
])
def test_attention_shape_validation(lib, kw, status):
    s = attn_shape(**kw)
    assert lib.moe_gqa_attention(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None) == status
    assert lib.moe_attention_workspace_size(ctypes.byref(s)) == 0


def test_attention_block_validation(lib):
    s = attn_shape()
    call = lambda **kw: lib.moe_attention_block_forward(
        ctypes.byref(s), kw.get("h", FAKE), FAKE, kw.get("eps", 1e-5), FAKE, FAKE, kw.get("theta", 1e6),
        kw.get("pos0", 0), FAKE, kw.get("ws_bytes", 1 << 40), None)
    assert call(eps=0.0) == _lib.MOE_ERR_INVALID_ARG and b"eps" in lib.moe_last_error()
    assert call(theta=0.0) == _lib.MOE_ERR_INVALID_ARG and b"rope_theta" in lib.moe_last_error()
    assert call(pos0=-1) == _lib.MOE_ERR_INVALID_ARG
    assert call(h=None) == _lib.MOE_ERR_INVALID_ARG and b"h_inout" in lib.moe_last_error()
    assert call(h=MISALIGNED) == _lib.MOE_ERR_INVALID_ARG
    assert call(ws_bytes=1024) == _lib.MOE_ERR_INVALID_ARG and b"workspace" in lib.moe_last_error()
    s0 = attn_shape(T=0)
    assert lib.moe_attention_block_forward(ctypes.byref(s0), FAKE, FAKE, 1e-5, FAKE, FAKE, 1e6, 0, None, 0,
                                           None) == _lib.MOE_OK
    assert lib.moe_gqa_attention(ctypes.byref(s0), None, None, None, None, None) == _lib.MOE_OK


def test_attention_workspace_size(lib):
    d, H, G, dh = 4096, 32, 8, 128

    def need(T):  # normalised input, q, k, v, o (bf16)
        return T * d * 2 + T * H * dh * 2 * 2 + T * G * dh * 2 * 2

    # GEMM path: partial sums and the RoPE (cos, sin) table [T][64]; neither
    # fp32 projection (RoPE and the residual add run in the GEMM epilogues).
    ws = lib.moe_attention_workspace_size(ctypes.byref(attn_shape(T=4096, d=d, H=H, G=G, d_h=dh)))
    gemm = need(4096) + 4096 * 64 * 8 + GEMM_PARTIALS
    assert gemm <= ws < gemm + (1 << 20)
    # Streaming path (T <= 64): the fp32 Q|K|V and output projections, no
    # partials, no table.
    ws = lib.moe_attention_workspace_size(ctypes.byref(attn_shape(T=16, d=d, H=H, G=G, d_h=dh)))
    stream = need(16) + 16 * (H + 2 * G) * dh * 4 + 16 * d * 4
    assert stream <= ws < stream + 4096


def test_c99_client_compiles_links_and_runs(tmp_path):
    """The header is plain C: a C99 client builds with -pedantic -Werror,
    links against libmoe.so and gets the host-side answers and errors."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libmoe.so not built")
    exe = str(tmp_path / "abi_client")
    src = os.path.join(ROOT, "tests", "c_client", "abi_client.c")
    build = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                            os.path.join(ROOT, "include"), src, "-L", lib_dir, "-lmoe",
                            f"-Wl,-rpath,{lib_dir}", "-o", exe], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    assert "k = 9 rejected" in run.stdout


# ---------------------------------------------------------------------------
# the binding's layout checks (host logic on CPU tensors: the C ABI sees only
# pointers, so a mis-shaped tensor must be refused before any call)
# ---------------------------------------------------------------------------
def _weights(E=4, d=64, d_ff=128, dt=torch.bfloat16):
    return (torch.zeros(E, d, dtype=torch.float32), torch.zeros(E, dtype=torch.float32),
            torch.zeros(E, d_ff, d, dtype=dt), torch.zeros(E, d_ff, d, dtype=dt), torch.zeros(E, d, d_ff, dtype=dt))


def test_binding_accepts_the_stated_layouts():
    w_gate, bias, w1, w3, w2 = _weights()
    assert moe._layer_weights(64, w_gate, bias, w1, w3, w2) == (4, 128)
    assert moe._layer_weights(64, None, None, w1, w3, w2) == (4, 128)
    moe._rows(torch.zeros(10, dtype=torch.int32), "st", torch.int32, 10)
    moe._rows(torch.zeros(12, 64, dtype=torch.float32), "ys", torch.float32, 10, 64)


@pytest.mark.parametrize("bad", ["w_gate_bf16", "w_gate_rows", "bias_len", "w3_shape", "w2_transposed",
                                 "w2_dtype", "w1_2d", "width"])
def test_binding_refuses_mis_shaped_weights(bad):
    w_gate, bias, w1, w3, w2 = _weights()
    d = 64
    if bad == "w_gate_bf16":
        w_gate = w_gate.to(torch.bfloat16)
    elif bad == "w_gate_rows":
        w_gate = torch.zeros(8, 64, dtype=torch.float32)
    elif bad == "bias_len":
        bias = torch.zeros(8, dtype=torch.float32)
    elif bad == "w3_shape":
        w3 = torch.zeros(4, 64, 64, dtype=torch.bfloat16)
    elif bad == "w2_transposed":
        w2 = torch.zeros(4, 128, 64, dtype=torch.bfloat16)
    elif bad == "w2_dtype":
        w2 = w2.to(torch.float32)
    elif bad == "w1_2d":
        w1 = torch.zeros(4 * 128, 64, dtype=torch.bfloat16)
    elif bad == "width":
        d = 128
    with pytest.raises(ValueError):
        moe._layer_weights(d, w_gate, bias, w1, w3, w2)


def test_binding_refuses_short_row_buffers():
    with pytest.raises(ValueError):
        moe._rows(torch.zeros(9, dtype=torch.int32), "sorted_token", torch.int32, 10)
    with pytest.raises(ValueError):
        moe._rows(torch.zeros(10, 32, dtype=torch.float32), "y_sorted", torch.float32, 10, 64)
    with pytest.raises(ValueError):
        moe._rows(torch.zeros(10, 64, dtype=torch.bfloat16), "y_sorted", torch.float32, 10, 64)
    with pytest.raises(ValueError):
        moe._need(torch.zeros(16, 64, dtype=torch.float32), "out", torch.bfloat16, (16, 64))
    with pytest.raises(ValueError):
        moe._activations(torch.zeros(2, 16, 64))
