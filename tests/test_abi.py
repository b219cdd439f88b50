"""The C ABI without a GPU: symbols, constants, argument validation (which runs before any HIP call),
workspace sizing, and the library's own host-side Philox against the oracle's."""

import ctypes
import os
import re

import numpy as np
import pytest

import stochastic_sparse_attention_split_amd as santa
from oracle import philox

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "santa.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(santa.LIB_PATH):
        from stochastic_sparse_attention_split_amd import _build
        _build.build()
    return santa.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(santa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert set(names) == set(santa.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_header_constants_match_binding():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define\s+(SANTA_[A-Z0-9_]+)\s+(0x[0-9a-fA-F]+|\d+)", text))
    val = {k: int(v, 0) for k, v in defs.items()}
    assert val["SANTA_IID"] == santa.IID and val["SANTA_STRAT"] == santa.STRAT and val["SANTA_SYS"] == santa.SYS
    assert val["SANTA_PROP"] == santa.PROP and val["SANTA_FLASH"] == santa.FLASH
    assert val["SANTA_TERNARY_Q"] == santa.TERNARY_Q
    assert val["SANTA_GROUP_BERNOULLI_Q"] == santa.GROUP_BERNOULLI_Q
    assert val["SANTA_K_FEATURE_MAJOR"] == santa.K_FEATURE_MAJOR
    assert val["SANTA_BF16"] == santa.BF16 and val["SANTA_F32"] == santa.F32
    assert val["SANTA_OK"] == santa.OK and val["SANTA_ERR_HIP"] == santa.ERR_HIP


def _args(**kw):
    a = santa.SantaArgs()
    base = dict(q=0x1000, K=0x2000, V=0x3000, out=0x4000, batch=1, heads=8, kv_heads=2, d=128, nk=1000, S=16,
                mode=santa.STRAT, dtype=santa.BF16, seed=1, workspace=0x5000, workspace_bytes=1 << 40)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), santa.ERR_INVALID_ARG),
    (dict(out=0), santa.ERR_INVALID_ARG),
    (dict(heads=6, kv_heads=4), santa.ERR_INVALID_ARG),
    (dict(S=0), santa.ERR_INVALID_ARG),
    (dict(nk=0), santa.ERR_INVALID_ARG),
    (dict(batch=0), santa.ERR_INVALID_ARG),
    (dict(mode=5), santa.ERR_INVALID_ARG),
    (dict(mode=santa.STRAT | santa.GROUP_BERNOULLI_Q, bern_samples=4), santa.ERR_INVALID_ARG),  # needs K^T
    (dict(mode=santa.STRAT | santa.GROUP_BERNOULLI_Q | santa.K_FEATURE_MAJOR | santa.TERNARY_Q, bern_samples=4),
     santa.ERR_INVALID_ARG),
    (dict(mode=santa.STRAT | santa.GROUP_BERNOULLI_Q | santa.K_FEATURE_MAJOR, bern_samples=0), santa.ERR_INVALID_ARG),
    (dict(mode=santa.STRAT | santa.GROUP_BERNOULLI_Q | santa.K_FEATURE_MAJOR, bern_samples=65),
     santa.ERR_INVALID_ARG),
    (dict(mode=santa.STRAT | santa.K_FEATURE_MAJOR, kt_row_stride=992), santa.ERR_INVALID_ARG),  # < nk
    (dict(mode=santa.STRAT | santa.K_FEATURE_MAJOR, kt_row_stride=1012), santa.ERR_INVALID_ARG),  # 2024 B rows
    (dict(mode=santa.STRAT | santa.K_FEATURE_MAJOR, batch=2, kt_batch_stride=8), santa.ERR_INVALID_ARG),
    (dict(mode=0x200), santa.ERR_INVALID_ARG),
    (dict(d=96), santa.ERR_UNSUPPORTED),
    (dict(dtype=7), santa.ERR_UNSUPPORTED),
    (dict(heads=32, kv_heads=2), santa.ERR_UNSUPPORTED),
    (dict(nk=(1 << 20) + 1), santa.ERR_UNSUPPORTED),
    (dict(S=70000), santa.ERR_UNSUPPORTED),
    (dict(kv_seq_stride=100), santa.ERR_INVALID_ARG),
    (dict(kv_seq_stride=257), santa.ERR_INVALID_ARG),
    (dict(K=0x2008), santa.ERR_INVALID_ARG),
    (dict(batch=2, kv_batch_stride=256 * 999), santa.ERR_INVALID_ARG),
    (dict(workspace_bytes=100), santa.ERR_WORKSPACE),
    (dict(workspace=0), santa.ERR_WORKSPACE),
])
def test_validation_rejects_before_any_hip_call(L, kw, code):
    a = _args(**kw)
    assert L.santa_decode_ex(ctypes.byref(a)) == code
    assert santa.last_error() != ""


def test_null_args_and_dense_validation(L):
    assert L.santa_decode_ex(None) == santa.ERR_INVALID_ARG
    assert L.santa_dense_decode(None) == santa.ERR_INVALID_ARG
    a = _args(d=80)
    assert L.santa_dense_decode(ctypes.byref(a)) == santa.ERR_UNSUPPORTED
    a = _args(workspace_bytes=4)
    assert L.santa_dense_decode(ctypes.byref(a)) == santa.ERR_WORKSPACE
    # the simple entry point validates before it allocates
    assert L.santa_decode(None, None, None, 100, 8, 2, 128, 16, 1, 0, None) == santa.ERR_INVALID_ARG
    assert L.santa_decode(1, 1, 1, 100, 8, 2, 100, 16, 1, 0, 1) == santa.ERR_UNSUPPORTED


def test_stream_read_validation(L):
    """The bandwidth probe validates its arguments before any HIP call."""
    need = L.santa_stream_read_scratch_bytes()
    assert need >= 4 * 1024
    assert L.santa_stream_read(None, 1024, 4096, need, None, None) == santa.ERR_INVALID_ARG
    assert L.santa_stream_read(4096, 1024, None, need, None, None) == santa.ERR_INVALID_ARG
    assert L.santa_stream_read(4096, 1000, 8192, need, None, None) == santa.ERR_INVALID_ARG  # not a multiple of 16
    assert L.santa_stream_read(4104, 1024, 8192, need, None, None) == santa.ERR_INVALID_ARG  # src not 16-byte aligned
    assert L.santa_stream_read(4096, 0, 8192, need, None, None) == santa.ERR_INVALID_ARG
    assert L.santa_stream_read(4096, 1024, 8192, need - 4, None, None) == santa.ERR_WORKSPACE


def test_workspace_bytes(L):
    B, nk, H, Hkv, S = 2, 1000, 8, 2, 16
    T = (nk + 255) // 256
    n = santa.workspace_bytes(B, nk, H, Hkv, 128, S)
    G = H // Hkv
    assert n >= (B * H * nk * 8 + 3 * B * H * T * 8 + B * H * (T + 1) * 8 + B * H * 4
                 + B * Hkv * T * G * 128 * 4 + B * H * S * 4 + B * Hkv * T * 4)
    assert n % 256 == 0
    assert santa.workspace_bytes(1, 0, 8, 2, 128, S) == 0
    assert santa.workspace_bytes(1, 10, 6, 4, 128, S) == 0
    assert santa.workspace_bytes(1, 10, 8, 2, 96, S) == 0
    assert santa.dense_workspace_bytes(1, 1024, 8, 2, 128) >= 8 * 2 * 130 * 4
    assert santa.dense_workspace_bytes(1, 1024, 8, 2, 96) == 0


def test_samples_per_head(L):
    from oracle import flash
    for nk, S in [(1, 1), (256, 7), (1000, 16), (32768, 2048), (32768, 100), (300000, 512), (1 << 20, 65535)]:
        T = (nk + 255) // 256
        for m in ("iid", "strat", "sys", "prop"):
            assert santa.samples_per_head(nk, S, m) == S
        assert santa.samples_per_head(nk, S, "flash") == T * flash.tile_budget(S, T)
    assert L.santa_samples_per_head(0, 4, 1) == -1
    assert L.santa_samples_per_head(10, 0, 1) == -1
    assert L.santa_samples_per_head(10, 4, 5) == -1
    # the flash workspace holds the longer index list
    assert santa.workspace_bytes(1, 32768, 8, 2, 128, 100, "flash") >= santa.workspace_bytes(1, 32768, 8, 2, 128, 100)


def test_library_philox_matches_oracle(L):
    rng = np.random.default_rng(1)
    for _ in range(300):
        c = [int(x) for x in rng.integers(0, 2**32, 4)]
        k = [int(x) for x in rng.integers(0, 2**32, 2)]
        want = tuple(int(x) for x in philox.philox4x32_10(*c, *k))
        assert santa.philox4x32_10(c, k) == want


def test_library_exp_matches_libm(L):
    """The kernels' fp64 exponential (run here on the host through the same inline code) against Python's
    libm exp: within 4 units in the last place for normal results, within 2 denormal steps below them,
    exactly 1 at 0 and exactly 0 for -inf and below -746."""
    import math

    import numpy as np

    assert santa.exp_f64(0.0) == 1.0
    assert santa.exp_f64(-0.0) == 1.0
    assert santa.exp_f64(-math.inf) == 0.0
    assert santa.exp_f64(-746.5) == 0.0
    rng = np.random.default_rng(5)
    xs = np.concatenate([
        -np.linspace(0.0, 745.0, 20001),
        -rng.exponential(1.0, 20000),                    # the bulk of softmax arguments
        -np.logspace(-300, 2.8, 4000),                   # tiny and large magnitudes
        -np.log(2.0) * (np.arange(0, 1075) + 0.5),       # reduction boundaries (k + 1/2) ln2
        [-709.78, -708.4, -745.13, -744.4, -1e-17],
    ])
    worst = 0.0
    for x in xs:
        x = float(x)
        got, ref = santa.exp_f64(x), math.exp(x)
        if ref >= 2.0 ** -1022:
            err = abs(got - ref) / math.ulp(ref)
            worst = max(worst, err)
            assert err <= 4.0, (x, got, ref)
        else:
            assert abs(got - ref) <= 2 * 2.0 ** -1074, (x, got, ref)
    assert worst <= 4.0


def test_status_strings_and_version(L):
    assert santa.version().startswith("santa-mi355x")
    for s in range(5):
        assert L.santa_status_string(s)


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(santa, "_lib", None)
    monkeypatch.setattr(santa, "LIB_PATH", "/nonexistent/libsanta.so")
    with pytest.raises(RuntimeError):
        santa.lib()


def test_noalloc_validation_before_any_hip_call(L):
    """santa_decode_noalloc checks its arguments and the size of its static scratch before any HIP call."""
    assert L.santa_decode_noalloc(None) == santa.ERR_INVALID_ARG
    a = _args(heads=6, kv_heads=4)
    assert L.santa_decode_noalloc(ctypes.byref(a)) == santa.ERR_INVALID_ARG
    st = santa.SantaStats()
    a = _args(stats_out=ctypes.pointer(st))
    assert L.santa_decode_noalloc(ctypes.byref(a)) == santa.ERR_INVALID_ARG
    assert "debug" in santa.last_error()
    a = _args(stage_ms=(ctypes.c_float * 4)())
    assert L.santa_decode_noalloc(ctypes.byref(a)) == santa.ERR_INVALID_ARG
    # 8 sequences of 2^20 keys need far more than the scratch holds; workspace fields are ignored
    a = _args(batch=8, nk=1 << 20, heads=32, kv_heads=8, workspace=0, workspace_bytes=0)
    assert L.santa_decode_noalloc(ctypes.byref(a)) == santa.ERR_WORKSPACE
    assert "santa_decode_noalloc holds" in santa.last_error()
