"""Python binding of libsanta.so, the MI355X (gfx950) SANTA / S²ANTA decode-attention library.

Argument marshalling only: every step of the decode runs in the library's HIP kernels. PyTorch provides
device memory and the current stream. The entry points mirror include/santa.h:

    decode(q, K, V, S, mode, seed, ...)      -> santa_decode_ex
    decode_simple(q, K, V, S, mode, seed)    -> santa_decode (library-owned workspace, batch 1, bf16)
    decode_noalloc(q, K, V, S, mode, seed)   -> santa_decode_noalloc (the library's static device scratch)
    dense_decode(q, K, V, ...)               -> santa_dense_decode (dense baseline)
    workspace_bytes(...), dense_workspace_bytes(...), philox4x32_10(ctr, key), version(), last_error()

Shapes: q [B, H, d]; K, V [B, nk, Hkv, d] (the sequence dimension may be strided, e.g. a preallocated
cache with room for more positions); out [B, H, d]. dtype bf16 or fp32.

The library is built in-tree (``python -m stochastic_sparse_attention_split_amd._build`` or
``__graft_entry__.build()``); importing works without it, but every call raises if it is missing.
"""

from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsanta.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_TIMEOUT = 0, 1, 2, 3, 4, 5
IID, STRAT, SYS, PROP, FLASH = 0, 1, 2, 3, 4
TERNARY_Q = 0x100
GROUP_BERNOULLI_Q = 0x200
K_FEATURE_MAJOR = 0x400
MULTI_LAUNCH = 0x800
BF16, F32 = 0, 1
MODES = {"iid": IID, "strat": STRAT, "sys": SYS, "prop": PROP, "flash": FLASH}

EXPORTED = [
    "santa_decode", "santa_decode_ex", "santa_workspace_bytes", "santa_dense_decode",
    "santa_dense_workspace_bytes", "santa_philox4x32_10", "santa_exp_f64", "santa_status_string", "santa_last_error",
    "santa_version", "santa_release", "santa_samples_per_head", "santa_stream_read",
    "santa_stream_read_scratch_bytes", "santa_decode_noalloc", "santa_status",
]


class SantaStats(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int32), ("bytes_k", ctypes.c_int64), ("bytes_v", ctypes.c_int64),
                ("bytes_qo", ctypes.c_int64), ("unique_rows", ctypes.c_int64),
                ("group_unique_rows", ctypes.POINTER(ctypes.c_int64))]


class SantaArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("K", ctypes.c_void_p), ("V", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("d", ctypes.c_int32),
        ("nk", ctypes.c_int64), ("kv_seq_stride", ctypes.c_int64), ("kv_batch_stride", ctypes.c_int64),
        ("S", ctypes.c_int32), ("mode", ctypes.c_int32), ("dtype", ctypes.c_int32), ("bern_samples", ctypes.c_int32),
        ("seed", ctypes.c_uint64), ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("idx_out", ctypes.c_void_p), ("prob_out", ctypes.c_void_p),
        ("stats_out", ctypes.POINTER(SantaStats)), ("stage_ms", ctypes.POINTER(ctypes.c_float)),
        ("kt_row_stride", ctypes.c_int64), ("kt_batch_stride", ctypes.c_int64),
        ("debug_spin_limit", ctypes.c_int32),
    ]


class SantaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"santa status {status}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libsanta.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (stochastic_sparse_attention_split_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        L.santa_decode.restype = ctypes.c_int
        L.santa_decode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                   ctypes.c_void_p]
        L.santa_decode_ex.restype = ctypes.c_int
        L.santa_decode_ex.argtypes = [ctypes.POINTER(SantaArgs)]
        L.santa_decode_noalloc.restype = ctypes.c_int
        L.santa_decode_noalloc.argtypes = [ctypes.POINTER(SantaArgs)]
        L.santa_status.restype = ctypes.c_int
        L.santa_status.argtypes = [ctypes.POINTER(SantaArgs)]
        L.santa_dense_decode.restype = ctypes.c_int
        L.santa_dense_decode.argtypes = [ctypes.POINTER(SantaArgs)]
        L.santa_samples_per_head.restype = ctypes.c_int64
        L.santa_samples_per_head.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int]
        L.santa_workspace_bytes.restype = ctypes.c_size_t
        L.santa_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int]
        L.santa_dense_workspace_bytes.restype = ctypes.c_size_t
        L.santa_dense_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int]
        L.santa_exp_f64.restype = ctypes.c_double
        L.santa_exp_f64.argtypes = [ctypes.c_double]
        L.santa_philox4x32_10.restype = None
        L.santa_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32),
                                          ctypes.POINTER(ctypes.c_uint32)]
        L.santa_status_string.restype = ctypes.c_char_p
        L.santa_status_string.argtypes = [ctypes.c_int]
        L.santa_last_error.restype = ctypes.c_char_p
        L.santa_last_error.argtypes = []
        L.santa_version.restype = ctypes.c_char_p
        L.santa_version.argtypes = []
        L.santa_release.restype = None
        L.santa_release.argtypes = []
        L.santa_stream_read.restype = ctypes.c_int
        L.santa_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
        L.santa_stream_read_scratch_bytes.restype = ctypes.c_size_t
        L.santa_stream_read_scratch_bytes.argtypes = []
        _lib = L
    return _lib


def version() -> str:
    return lib().santa_version().decode()


def last_error() -> str:
    return lib().santa_last_error().decode()


def _check(status: int):
    if status != OK:
        raise SantaError(status, last_error() or lib().santa_status_string(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or fp32 expected")


def _mode_code(mode, ternary: bool) -> int:
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    return m | (TERNARY_Q if ternary else 0)


def samples_per_head(nk: int, S: int, mode=STRAT) -> int:
    """Sampled keys listed per head (the last dimension of idx_out): S, or T * S_tile for "flash"."""
    return int(lib().santa_samples_per_head(int(nk), int(S), _mode_code(mode, False)))


def workspace_bytes(B: int, nk: int, H: int, Hkv: int, d: int, S: int, mode=STRAT) -> int:
    return int(lib().santa_workspace_bytes(B, nk, H, Hkv, d, S, _mode_code(mode, False)))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace for decode(). No initial contents are required; it can be reused by later calls that do
    not overlap with each other."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def dense_workspace_bytes(B: int, nk: int, H: int, Hkv: int, d: int) -> int:
    return int(lib().santa_dense_workspace_bytes(B, nk, H, Hkv, d))


def feature_major(K: torch.Tensor) -> torch.Tensor:
    """K^T [B, Hkv, d, rows] from a sequence-major K [B, nk, Hkv, d]: feature rows of nk keys, padded with
    zeros to a multiple of 8 keys (the row stride the library needs). Returns a view of the padded tensor
    narrowed to nk keys; its stride(2) is the padded row stride."""
    B, nk, Hkv, d = K.shape
    rows = (nk + 7) // 8 * 8
    kt = torch.zeros((B, Hkv, d, rows), dtype=K.dtype, device=K.device)
    kt[..., :nk] = K.permute(0, 2, 3, 1)
    return kt[..., :nk]


def _fill_common(a: SantaArgs, q, K, V, out, nk, stream, k_feature_major: bool = False):
    if q.dim() != 3 or K.dim() != 4 or V.dim() != 4:
        raise ValueError("q must be [B, H, d]; K and V [B, nk, Hkv, d] (K^T [B, Hkv, d, nk] if feature-major)")
    kptr = K.data_ptr()
    if k_feature_major:
        if K.shape != (V.shape[0], V.shape[2], V.shape[3], V.shape[1]) or K.stride(3) != 1 \
                or K.stride(1) != K.shape[2] * K.stride(2):
            raise ValueError("feature-major K must be K^T [B, Hkv, d, nk] with unit key stride and packed rows")
        if K.dtype != V.dtype:
            raise TypeError("K and V must share one dtype")
        a.kt_row_stride = K.stride(2)
        a.kt_batch_stride = K.stride(0)
        K = V  # the remaining checks and the sequence strides are those of V
    if K.shape != V.shape or K.stride() != V.stride():
        raise ValueError("K and V must have the same shape and strides")
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous")
    if K.stride(3) != 1 or K.stride(2) != K.shape[3]:
        raise ValueError("K/V rows must be contiguous [Hkv, d] per position")
    if not (q.dtype == K.dtype == V.dtype == out.dtype):
        raise TypeError("q, K, V and out must share one dtype")
    B, H, d = q.shape
    a.q, a.K, a.V, a.out = q.data_ptr(), kptr, V.data_ptr(), out.data_ptr()
    a.batch, a.heads, a.kv_heads, a.d = B, H, K.shape[2], d
    a.nk = K.shape[1] if nk is None else int(nk)
    a.kv_seq_stride = K.stride(1)
    a.kv_batch_stride = K.stride(0)
    a.dtype = _dtype_code(q)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    a.stream = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _set_debug_outputs(a: SantaArgs, idx_out, prob_out):
    if idx_out is not None:
        L = int(lib().santa_samples_per_head(a.nk, a.S, a.mode))
        if idx_out.dtype != torch.int32 or idx_out.numel() < a.batch * a.heads * L:
            raise ValueError(f"idx_out must be int32 with batch*heads*{L} elements")
        a.idx_out = idx_out.data_ptr()
    if prob_out is not None:
        if prob_out.dtype != torch.float64 or prob_out.numel() < a.batch * a.heads * a.nk:
            raise ValueError("prob_out must be float64 with batch*heads*nk elements")
        a.prob_out = prob_out.data_ptr()


def decode(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, S: int, mode="strat", seed: int = 0, *,
           ternary: bool = False, nk: int | None = None, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, idx_out: torch.Tensor | None = None,
           prob_out: torch.Tensor | None = None, stats: bool = False, stage_ms: bool = False, stream=None,
           group_bernoulli: int = 0, k_feature_major: bool = False, multi_launch: bool = False,
           debug_spin_limit: int = 0):
    """One SANTA / S²ANTA decode step through santa_decode_ex.

    k_feature_major: K is K^T [B, Hkv, d, nk] (see feature_major()); group_bernoulli = B > 0 selects the
    mean-group-query Bernoulli scores with B stratified samples (feature-major K only); multi_launch forces
    the multi-launch path; debug_spin_limit > 0 bounds every in-kernel wait to that many polls.
    Returns out, or (out, info) when stats or stage_ms is requested (info holds the stats fields, the
    distinct sampled rows per (sequence, KV head) as "group_unique_rows", and the milliseconds [score,
    chunk CDF + resolve, merge, total] from events between the launches).
    """
    if out is None:
        out = torch.empty_like(q)
    a = SantaArgs()
    _fill_common(a, q, K, V, out, nk, stream, k_feature_major)
    a.S = int(S)
    a.mode = _mode_code(mode, ternary) | (K_FEATURE_MAJOR if k_feature_major else 0)
    a.mode |= MULTI_LAUNCH if multi_launch else 0
    if group_bernoulli:
        a.mode |= GROUP_BERNOULLI_Q
        a.bern_samples = int(group_bernoulli)
    a.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    a.debug_spin_limit = int(debug_spin_limit)
    need = int(lib().santa_workspace_bytes(a.batch, a.nk, a.heads, a.kv_heads, a.d, a.S, a.mode))
    if workspace is None:
        workspace = new_workspace(need, q.device)
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    _set_debug_outputs(a, idx_out, prob_out)
    st = SantaStats()
    ms = (ctypes.c_float * 4)()
    gu = (ctypes.c_int64 * (a.batch * a.kv_heads))()
    if stats:
        st.group_unique_rows = gu
        a.stats_out = ctypes.pointer(st)
    if stage_ms:
        a.stage_ms = ms
    _check(lib().santa_decode_ex(ctypes.byref(a)))
    if stats or stage_ms:
        info = {}
        if stats:
            info.update({f: getattr(st, f) for f, _ in SantaStats._fields_ if f != "group_unique_rows"})
            info["group_unique_rows"] = [int(x) for x in gu]
        if stage_ms:
            info["stage_ms"] = list(ms)
        return out, info
    return out


def status(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, S: int, mode="strat", *, workspace=None,
           nk: int | None = None, stream=None, k_feature_major: bool = False) -> int:
    """santa_status: the status code the last call with these sizes left in `workspace` (None: the scratch of
    santa_decode_noalloc). Synchronises the stream. Returns OK or ERR_TIMEOUT (no exception)."""
    a = SantaArgs()
    out = torch.empty_like(q)
    _fill_common(a, q, K, V, out, nk, stream, k_feature_major)
    a.S = int(S)
    a.mode = _mode_code(mode, False) | (K_FEATURE_MAJOR if k_feature_major else 0)
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return int(lib().santa_status(ctypes.byref(a)))


def decode_noalloc(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, S: int, mode="strat", seed: int = 0, *,
                   out: torch.Tensor, ternary: bool = False, nk: int | None = None,
                   idx_out: torch.Tensor | None = None, prob_out: torch.Tensor | None = None, stream=None,
                   group_bernoulli: int = 0, k_feature_major: bool = False):
    """One decode step through santa_decode_noalloc: the workspace is the library's own device array, so
    the call allocates nothing (``out`` must be given; no stats or stage timing)."""
    a = SantaArgs()
    _fill_common(a, q, K, V, out, nk, stream, k_feature_major)
    a.S = int(S)
    a.mode = _mode_code(mode, ternary) | (K_FEATURE_MAJOR if k_feature_major else 0)
    if group_bernoulli:
        a.mode |= GROUP_BERNOULLI_Q
        a.bern_samples = int(group_bernoulli)
    a.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    _set_debug_outputs(a, idx_out, prob_out)
    _check(lib().santa_decode_noalloc(ctypes.byref(a)))
    return out


def decode_simple(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, S: int, mode="strat", seed: int = 0, *,
                  ternary: bool = False, out: torch.Tensor | None = None):
    """santa_decode: batch 1, bf16, contiguous caches, default stream, library-owned workspace."""
    if out is None:
        out = torch.empty_like(q)
    if q.dim() == 3:
        if q.shape[0] != 1:
            raise ValueError("santa_decode takes batch 1")
        q1, K1, V1 = q[0], K[0], V[0]
    else:
        q1, K1, V1 = q, K, V
    for t in (q1, K1, V1, out):
        if not t.is_contiguous():
            raise ValueError("santa_decode needs contiguous tensors")
    nk, Hkv, d = K1.shape
    H = q1.shape[0]
    _check(lib().santa_decode(q1.data_ptr(), K1.data_ptr(), V1.data_ptr(), nk, H, Hkv, d, int(S),
                              _mode_code(mode, ternary), int(seed) & 0xFFFFFFFFFFFFFFFF, out.data_ptr()))
    return out


def dense_decode(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, *, nk: int | None = None,
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Dense decode attention baseline through santa_dense_decode."""
    if out is None:
        out = torch.empty_like(q)
    a = SantaArgs()
    _fill_common(a, q, K, V, out, nk, stream)
    need = int(lib().santa_dense_workspace_bytes(a.batch, a.nk, a.heads, a.kv_heads, a.d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().santa_dense_decode(ctypes.byref(a)))
    return out


def stream_read(t: torch.Tensor, scratch: torch.Tensor | None = None, stream=None, kernel_time: bool = False):
    """Reads the bytes of a contiguous device tensor once through santa_stream_read (a bandwidth probe);
    returns the scratch tensor holding one XOR word per block, or (scratch, kernel milliseconds) with
    kernel_time (events HIP records with the launch: its dispatch and execution; synchronises)."""
    if not t.is_contiguous():
        raise ValueError("stream_read needs a contiguous tensor")
    need = int(lib().santa_stream_read_scratch_bytes())
    if scratch is None:
        scratch = torch.empty(need, dtype=torch.uint8, device=t.device)
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    st = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    ms = ctypes.c_float(0.0)
    _check(lib().santa_stream_read(t.data_ptr(), t.numel() * t.element_size(), scratch.data_ptr(),
                                   scratch.numel() * scratch.element_size(), st,
                                   ctypes.byref(ms) if kernel_time else None))
    return (scratch, float(ms.value)) if kernel_time else scratch


def philox4x32_10(ctr, key):
    """The library's own host-side Philox4x32-10 (the kernels' code path) -> 4 uint32 words."""
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (ctypes.c_uint32 * 4)()
    lib().santa_philox4x32_10(c, k, o)
    return tuple(int(x) for x in o)


def exp_f64(x: float) -> float:
    """The library's own fp64 exponential evaluated on the host (the kernels' code path)."""
    return float(lib().santa_exp_f64(float(x)))


def release():
    lib().santa_release()
