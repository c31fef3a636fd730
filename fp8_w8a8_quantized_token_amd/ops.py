"""Torch-facing wrappers over the C ABI (marshalling only).

torch provides device memory and the current HIP stream; every computation
runs in the library's gfx950 kernels. FP8 tensors are raw OCP E4M3 codes held
as ``torch.uint8`` (``torch.float8_e4m3fn`` tensors are accepted and viewed as
bytes).

User-facing calls mirror the pages' functions:
* ``linear_channelwise`` -- the channelwise branch of ``apply_fp8_linear``
  (PR 34331 digest, "Key source excerpts"): per-token activation quant, then
  the scaled GEMM with per-channel weight scales and a fused bias.
* ``quant_per_token_group`` -- the row-padded per-token-group quant (PR 27896
  digest, "Key source excerpts"): returns codes [M_pad, K] and scales as an
  [M_pad, K/G] view of [K/G, M_pad] storage.
* ``linear_blockwise`` -- the blockwise linear of the same digest, with the
  row slice and the bias folded into the GEMM's epilogue.
* ``silu_mul_quant_per_token(_group)``, ``scale_ue8m0=True`` -- the quantizer
  flags that digest's kernel call names (fuse_silu_and_mul, scale_ue8m0).
* ``quant_static`` -- the static per-tensor quantization named by the PR 31340
  digest ("Fix FP8 Triton dtype selection on A100", "Implementation").
"""
import ctypes
import threading

import torch

from . import _lib
from ._lib import KIND_BLOCKWISE, KIND_CHANNELWISE, TileConfig, VARIANTS, check

__all__ = [
    "prepare", "padded_rows", "quant_per_token", "quant_per_token_group", "silu_mul_quant_per_token",
    "silu_mul_quant_per_token_group", "quant_static", "masked_quant_per_token_group",
    "scaled_mm_blockwise_masked", "scaled_mm_channelwise",
    "scaled_mm_blockwise", "linear_channelwise", "linear_blockwise", "tile_config",
    "default_tile_config", "set_config_dir", "workspace_bytes", "make_config", "linear_launches",
]


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _as_codes(t, name):
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn), got {t.dtype}")
    return t


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def make_config(variant, split_k=1):
    """TileConfig for an explicit kernel variant name (see _lib.VARIANTS)."""
    return TileConfig(VARIANTS[variant] if isinstance(variant, str) else int(variant), 0, 0, 0,
                      int(split_k), 0)


# ---------------------------------------------------------------- workspace
class _WorkspacePool:
    """One zero-filled split-K workspace per (device, stream), grown on demand.
    The kernels leave the arrival counters at zero after every call."""

    def __init__(self):
        self._lock = threading.Lock()
        self._bufs = {}

    def get(self, device, nbytes):
        if nbytes == 0:
            return None
        key = (device, torch.cuda.current_stream(device).cuda_stream)
        with self._lock:
            buf = self._bufs.get(key)
            if buf is None or buf.numel() < nbytes:
                size = max(nbytes, 1 << 20)
                buf = torch.zeros(size, dtype=torch.uint8, device=device)
                self._bufs[key] = buf
            return buf


_ws = _WorkspacePool()


def workspace_bytes(kind, m, n, k, config=None):
    cfg = ctypes.byref(config) if config is not None else None
    v = _lib.load().fp8_scaled_mm_workspace_size(kind, m, n, k, cfg)
    if v == ctypes.c_size_t(-1).value:
        raise ValueError("invalid arguments for workspace size")
    return v


# ---------------------------------------------------------------- quantization
def padded_rows(m, row_alignment=4):
    v = _lib.load().fp8_padded_rows(m, row_alignment)
    if v < 0:
        raise ValueError("invalid M or row_alignment")
    return v


def _quant_input(x, silu_mul):
    """Validate a quantizer input; returns K (the quantized row width)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise TypeError("x must be a 2-D bf16 tensor")
    _need_cuda(x)
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    k = x.shape[1]
    if silu_mul:
        if k % 2 != 0:
            raise ValueError("a SiLU-and-mul input holds [gate | up]: an even number of columns")
        k //= 2
    return k


def _flags(silu_mul, scale_ue8m0):
    return (_lib.QUANT_FUSE_SILU_MUL if silu_mul else 0) | (_lib.QUANT_SCALE_UE8M0 if scale_ue8m0 else 0)


def quant_per_token(x, eps=1e-10, out=None, scale=None, silu_mul=False, scale_ue8m0=False):
    """bf16 [M, K] -> (E4M3 codes uint8 [M, K], fp32 scales [M]).

    silu_mul: x is [M, 2K] = [gate | up] and the quantized row is
    bf16(silu(gate) * up); scale_ue8m0: scales rounded up to powers of two."""
    k = _quant_input(x, silu_mul)
    m = x.shape[0]
    q = out if out is not None else torch.empty((m, k), dtype=torch.uint8, device=x.device)
    s = scale if scale is not None else torch.empty((m,), dtype=torch.float32, device=x.device)
    check(_lib.load().fp8_quant_per_token_ex(_p(x), m, k, x.stride(0), _p(q), q.stride(0), _p(s),
                                             float(eps), _flags(silu_mul, scale_ue8m0), _stream(x)))
    return q, s


def quant_per_token_group(x, group_size=128, eps=1e-10, row_alignment=4, out=None,
                          scale_storage=None, silu_mul=False, scale_ue8m0=False):
    """bf16 [M, K] -> (codes uint8 [M_pad, K], scales fp32 [M_pad, K/G] with
    stride (1, M_pad)). Rows M..M_pad-1 of both are left unwritten.
    silu_mul / scale_ue8m0 as for quant_per_token."""
    k = _quant_input(x, silu_mul)
    m = x.shape[0]
    if group_size <= 0 or k % group_size != 0:
        raise ValueError("the last dimension of x must be divisible by group_size")
    m_pad = padded_rows(m, row_alignment)
    q = out if out is not None else torch.empty((m_pad, k), dtype=torch.uint8, device=x.device)
    st = scale_storage if scale_storage is not None else torch.empty(
        (k // group_size, m_pad), dtype=torch.float32, device=x.device)
    check(_lib.load().fp8_quant_per_token_group_ex(_p(x), m, k, x.stride(0), group_size,
                                                   row_alignment, _p(q), q.stride(0), _p(st),
                                                   float(eps), _flags(silu_mul, scale_ue8m0),
                                                   _stream(x)))
    return q, st.transpose(0, 1)


def silu_mul_quant_per_token(x, eps=1e-10, out=None, scale=None):
    """[gate | up] bf16 [M, 2K] -> per-token codes [M, K] and scales [M] of
    bf16(silu(gate) * up), in one pass over x."""
    return quant_per_token(x, eps, out, scale, silu_mul=True)


def silu_mul_quant_per_token_group(x, group_size=128, eps=1e-10, row_alignment=4, out=None,
                                   scale_storage=None, scale_ue8m0=False):
    """[gate | up] bf16 [M, 2K] -> row-padded group codes and column-major
    scales (as quant_per_token_group) of bf16(silu(gate) * up)."""
    return quant_per_token_group(x, group_size, eps, row_alignment, out, scale_storage,
                                 silu_mul=True, scale_ue8m0=scale_ue8m0)


def masked_quant_per_token_group(x, masked_m, group_size=128, eps=1e-10, row_alignment=4, out=None,
                                 scale_storage=None, silu_mul=False, scale_ue8m0=False):
    """MoE experts: x bf16 [E, M_max, K] (or [E, M_max, 2K] = [gate | up] with
    silu_mul), masked_m int32 [E] on the device (valid rows per expert) ->
    (codes uint8 [E, M_pad, K], scales fp32 [E, M_pad, K/G] as a view of
    [E, K/G, M_pad] storage). Rows at or beyond masked_m[e] are left unwritten."""
    if x.dtype != torch.bfloat16 or x.dim() != 3:
        raise TypeError("x must be a 3-D bf16 tensor [E, M_max, K]")
    _need_cuda(x, masked_m)
    if x.stride(2) != 1 or x.stride(0) != x.shape[1] * x.stride(1):
        raise ValueError("x must hold contiguous rows and expert slabs of M_max rows")
    if masked_m.dtype != torch.int32 or masked_m.numel() != x.shape[0] or not masked_m.is_contiguous():
        raise TypeError("masked_m must be a contiguous int32 tensor of E counts")
    e_n, m_max, k = x.shape
    if silu_mul:
        if k % 2:
            raise ValueError("a SiLU-and-mul input holds [gate | up]: an even number of columns")
        k //= 2
    if group_size <= 0 or k % group_size != 0:
        raise ValueError("the last dimension of x must be divisible by group_size")
    m_pad = padded_rows(m_max, row_alignment)
    q = out if out is not None else torch.empty((e_n, m_pad, k), dtype=torch.uint8, device=x.device)
    st = scale_storage if scale_storage is not None else torch.empty(
        (e_n, k // group_size, m_pad), dtype=torch.float32, device=x.device)
    if q.shape != (e_n, m_pad, k) or not q.is_contiguous() or st.shape != (e_n, k // group_size, m_pad) \
            or not st.is_contiguous():
        raise ValueError("out must be [E, M_pad, K] and scale_storage [E, K/G, M_pad], contiguous")
    check(_lib.load().fp8_quant_per_token_group_masked(
        _p(x), e_n, m_max, k, x.stride(1), _p(masked_m), group_size, row_alignment, _p(q), k, _p(st),
        float(eps), _flags(silu_mul, scale_ue8m0), _stream(x)))
    return q, st.transpose(1, 2)


def scaled_mm_blockwise_masked(a, b, a_scale, b_scale, masked_m, m_max=None, out=None, config=None,
                               scale_ue8m0=False):
    """Grouped blockwise GEMM over E experts: a codes [E, M_pad, K], a_scale an
    [E, M_pad, K/128] view of [E, K/128, M_pad] storage (as returned by
    masked_quant_per_token_group), b codes [E, N, K], b_scale fp32
    [E, N/128, K/128], masked_m int32 [E] on the device -> bf16 [E, M_max, N]
    whose rows at or beyond masked_m[e] are left unwritten (m_max defaults
    to M_pad)."""
    a = _as_codes(a, "a")
    b = _as_codes(b, "b")
    _need_cuda(a, b, a_scale, b_scale, masked_m)
    e_n, m_pad, k = a.shape
    n = b.shape[1]
    m_max = m_pad if m_max is None else int(m_max)
    if b.shape != (e_n, n, k) or not a.is_contiguous() or not b.is_contiguous():
        raise ValueError("a [E, M_pad, K] and b [E, N, K] must be contiguous and agree on E and K")
    if a_scale.dtype != torch.float32 or b_scale.dtype != torch.float32:
        raise TypeError("scales must be fp32")
    if a_scale.shape != (e_n, m_pad, k // 128) or a_scale.stride() != ((k // 128) * m_pad, 1, m_pad):
        raise ValueError("a_scale must be an [E, M_pad, K/128] view of [E, K/128, M_pad] storage")
    if b_scale.shape != (e_n, n // 128, k // 128) or not b_scale.is_contiguous():
        raise ValueError("b_scale must be contiguous [E, N/128, K/128]")
    if masked_m.dtype != torch.int32 or masked_m.numel() != e_n or not masked_m.is_contiguous():
        raise TypeError("masked_m must be a contiguous int32 tensor of E counts")
    if out is None:
        out = torch.empty((e_n, m_max, n), dtype=torch.bfloat16, device=a.device)
    if out.shape != (e_n, m_max, n) or not out.is_contiguous():
        raise ValueError("out must be contiguous [E, M_max, N]")
    cfg = config if config is not None else TileConfig(-1, 0, 0, 0, 1, 0)
    check(_lib.load().fp8_scaled_mm_blockwise_masked(
        _p(a), _p(b), _p(a_scale), m_pad, _p(b_scale), _p(out), _p(masked_m), e_n, m_max, n, k, k, k,
        n, 1 if scale_ue8m0 else 0, ctypes.byref(cfg), _stream(a)))
    return out


def quant_static(x, scale, out=None):
    """bf16 [M, K] and a given fp32 scale (a 1-element device tensor, positive
    and finite) -> E4M3 codes uint8 [M, K]; no scale is produced."""
    k = _quant_input(x, False)
    m = x.shape[0]
    _need_cuda(scale)
    if scale.dtype != torch.float32 or scale.numel() != 1:
        raise TypeError("scale must be a 1-element fp32 tensor")
    q = out if out is not None else torch.empty((m, k), dtype=torch.uint8, device=x.device)
    check(_lib.load().fp8_quant_static(_p(x), m, k, x.stride(0), _p(scale), _p(q), q.stride(0),
                                       _stream(x)))
    return q


# ---------------------------------------------------------------- GEMMs
def scaled_mm_channelwise(a, b, a_scale, b_scale, bias=None, out=None, config=None):
    """a codes [M, K], b codes [N, K] (K-contiguous), a_scale fp32 [M],
    b_scale fp32 [N], bias bf16 [N] or None -> bf16 [M, N]."""
    a = _as_codes(a, "a")
    b = _as_codes(b, "b")
    _need_cuda(a, b, a_scale, b_scale, bias)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k:
        raise ValueError("a and b disagree on K")
    if a_scale.dtype != torch.float32 or b_scale.dtype != torch.float32:
        raise TypeError("scales must be fp32")
    if a_scale.numel() < m or b_scale.numel() < n or not a_scale.is_contiguous() or \
            not b_scale.is_contiguous():
        raise ValueError("a_scale [M] and b_scale [N] must be contiguous")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() < n or
                             not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bf16 [N] tensor")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    cfg = config if config is not None else TileConfig(-1, 0, 0, 0, 1, 0)
    nws = workspace_bytes(KIND_CHANNELWISE, m, n, k, cfg)
    ws = _ws.get(a.device, nws)
    check(_lib.load().fp8_scaled_mm_channelwise_ex(
        _p(a), _p(b), _p(a_scale), _p(b_scale), _p(bias), _p(out), m, n, k, a.stride(0),
        b.stride(0), out.stride(0), _p(ws), nws, ctypes.byref(cfg), _stream(a)))
    return out


def scaled_mm_blockwise(a, b, a_scale, b_scale, bias=None, m=None, out=None, config=None,
                        scale_ue8m0=False):
    """a codes [>=M, K]; b codes [N, K]; a_scale an [M_pad, K/128] view with
    stride(0) == 1 (as returned by quant_per_token_group); b_scale fp32
    [N/128, K/128]; only the first m rows (default: all of a) are computed.
    scale_ue8m0: every scale is a power of two (the quantizers' scale_ue8m0
    output); the large-M tile then applies them inside the block-scaled MFMA."""
    a = _as_codes(a, "a")
    b = _as_codes(b, "b")
    _need_cuda(a, b, a_scale, b_scale, bias)
    m = a.shape[0] if m is None else int(m)
    k = a.shape[1]
    n = b.shape[0]
    if b.shape[1] != k:
        raise ValueError("a and b disagree on K")
    if a_scale.dtype != torch.float32 or b_scale.dtype != torch.float32:
        raise TypeError("scales must be fp32")
    if a_scale.dim() != 2 or a_scale.stride(0) != 1:
        raise ValueError("a_scale must be column-major ([M_pad, K/128] with stride(0) == 1)")
    if not b_scale.is_contiguous():
        raise ValueError("b_scale must be contiguous [N/128, K/128]")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() < n or
                             not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bf16 [N] tensor")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    cfg = config if config is not None else TileConfig(-1, 0, 0, 0, 1, 0)
    nws = workspace_bytes(KIND_BLOCKWISE, m, n, k, cfg)
    ws = _ws.get(a.device, nws)
    lib = _lib.load()
    fn = lib.fp8_scaled_mm_blockwise_ue8m0_ex if scale_ue8m0 else lib.fp8_scaled_mm_blockwise_ex
    check(fn(_p(a), _p(b), _p(a_scale), a_scale.stride(1), _p(b_scale), _p(bias), _p(out), m, n, k,
             a.stride(0), b.stride(0), out.stride(0), _p(ws), nws, ctypes.byref(cfg), _stream(a)))
    return out


# ---------------------------------------------------------------- linears
def _linear_args(kind, x, w_q, w_s, bias, eps, row_alignment, config, out, q, scale, flags=0):
    """Validated ctypes argument tuple of fp8_linear_{channelwise,blockwise}_ex
    for 2-D x (rows of 2K [gate | up] values under the SiLU-and-mul flag), plus
    the tensors it points to."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise TypeError("x must be a 2-D bf16 tensor with contiguous rows")
    w_q = _as_codes(w_q, "w_q")
    _need_cuda(x, w_q, w_s, bias)
    m, k = x.shape
    if flags & _lib.QUANT_FUSE_SILU_MUL:
        if k % 2:
            raise ValueError("the SiLU-and-mul input needs an even row width [gate | up]")
        k //= 2
    n = w_q.shape[0]
    if w_q.shape[1] != k:
        raise ValueError("x and w_q disagree on K")
    if w_s.dtype != torch.float32 or not w_s.is_contiguous():
        raise ValueError("w_s must be a contiguous fp32 tensor")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() < n or
                             not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bf16 [N] tensor")
    dev = x.device
    if kind == KIND_CHANNELWISE:
        m_pad = m
        q = q if q is not None else torch.empty((m, k), dtype=torch.uint8, device=dev)
        scale = scale if scale is not None else torch.empty((m,), dtype=torch.float32, device=dev)
    else:
        m_pad = padded_rows(m, row_alignment)
        q = q if q is not None else torch.empty((m_pad, k), dtype=torch.uint8, device=dev)
        scale = scale if scale is not None else torch.empty((k // 128, m_pad), dtype=torch.float32,
                                                            device=dev)
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    cfg = config if config is not None else TileConfig(-1, 0, 0, 0, 1, 0)
    nws = workspace_bytes(kind, m, n, k, cfg)
    ws = _ws.get(dev, nws)
    head = (_p(x), _p(w_q), _p(w_s), _p(bias), _p(out), m, n, k, x.stride(0), w_q.stride(0),
            out.stride(0))
    mid = (ctypes.c_float(eps),) if kind == KIND_CHANNELWISE else (row_alignment, ctypes.c_float(eps))
    args = (head + mid + (_p(q), q.stride(0), _p(scale), _p(ws), nws, ctypes.byref(cfg), flags,
                          _stream(x)))
    return args, (out, q, scale, cfg, ws)


def linear_channelwise(x, w_q, w_s, bias=None, eps=1e-10, config=None, return_quant=False,
                       silu_mul=False, scale_ue8m0=False):
    """y = x @ W^T with per-token FP8 activation quant and per-channel weight
    scales. x bf16 [..., K]; w_q codes [N, K]; w_s fp32 [N]; bias bf16 [N].
    One kernel launch for M <= 4 (quant fused into the skinny GEMM), two
    otherwise. return_quant=True also returns the codes [M, K] and scales [M].
    silu_mul=True: x is [..., 2K] = [gate | up] and the quantized row is
    SiLU(gate) * up rounded to bf16 (the down projection after a gated MLP);
    scale_ue8m0=True: power-of-two activation scales. The single launch takes
    UE8M0 up to M = 4 and SiLU-and-mul at M = 1 (blockwise: M <= 2)."""
    shape = x.shape
    x2 = x.reshape(-1, shape[-1])
    args, (out, q, s, _, _) = _linear_args(KIND_CHANNELWISE, x2, w_q, w_s, bias, eps, 1, config,
                                          None, None, None, _flags(silu_mul, scale_ue8m0))
    check(_lib.load().fp8_linear_channelwise_ex(*args))
    out = out.view(*shape[:-1], out.shape[1])
    return (out, q, s) if return_quant else out


def linear_blockwise(x, w_q, w_s, bias=None, block_size=(128, 128), eps=1e-10,
                     row_alignment=4, config=None, return_quant=False, silu_mul=False,
                     scale_ue8m0=False):
    """Blockwise FP8 linear: group-128 activation quant into row-padded buffers,
    then the blockwise GEMM over the first M rows with the bias fused. One
    launch for M <= 4, two otherwise. return_quant=True also returns the codes
    [M_pad, K] and the scales as an [M_pad, K/128] view of [K/128, M_pad].
    silu_mul as for linear_channelwise; scale_ue8m0=True makes the activation
    scales powers of two and runs the GEMM on the block-scaled MFMA tiles (the
    weight block scales must then be powers of two too)."""
    if tuple(block_size) != (128, 128):
        raise _lib.Fp8Error(_lib.FP8_ERR_UNSUPPORTED, "only 128x128 weight blocks are supported")
    shape = x.shape
    x2 = x.reshape(-1, shape[-1])
    args, (out, q, st, _, _) = _linear_args(KIND_BLOCKWISE, x2, w_q, w_s, bias, eps, row_alignment,
                                           config, None, None, None, _flags(silu_mul, scale_ue8m0))
    check(_lib.load().fp8_linear_blockwise_ex(*args))
    out = out.view(*shape[:-1], out.shape[1])
    return (out, q, st.transpose(0, 1)) if return_quant else out


def linear_launches(kind, m, n, k, config=None, silu_mul=False, scale_ue8m0=False):
    """Kernel launches one linear call makes: 1 (fused), 2, or 0 for M == 0."""
    cfg = ctypes.byref(config) if config is not None else None
    r = _lib.load().fp8_linear_launches_ex(kind, m, n, k, cfg, _flags(silu_mul, scale_ue8m0))
    if r < 0:
        check(r)
    return r


# ---------------------------------------------------------------- tile table
def tile_config(kind, n, k, m):
    """(config dict, hit) for the table lookup of (kind, N, K, M)."""
    c = TileConfig()
    r = _lib.load().fp8_tile_config_lookup(kind, n, k, m, ctypes.byref(c))
    if r < 0:
        check(r)
    return c.as_dict(), bool(r == 1)


def default_tile_config(kind, n, k, m):
    c = TileConfig()
    check(_lib.load().fp8_tile_config_default(kind, n, k, m, ctypes.byref(c)))
    return c.as_dict()


def set_config_dir(path):
    _lib.load().fp8_tile_config_set_dir(None if path is None else str(path).encode())


# ---------------------------------------------------------------- prepared launches
class Prepared:
    """A launch with every argument resolved up front: calling it is one ctypes
    call on the stream that was current when it was prepared. For hot loops
    whose tensors and shapes do not change (the benchmark, serving loops).
    The ctypes arguments are raw device pointers, so the object holds a
    reference to every tensor (and config struct) they point into: the
    memory stays allocated for as long as the launch can be called, also when
    the caller drops its own references or torch empties its cache."""

    def __init__(self, fn, args, name, keep):
        self._fn, self._args, self.name = fn, args, name
        self._keep = tuple(keep)

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            check(st)


def prepare(op, *args, **kwargs):
    """prepare("quant_per_token", x, out=q, scale=s), prepare("quant_per_token_group",
    x, group_size, row_alignment=4, out=q, scale_storage=st) (both also as
    "silu_mul_quant_per_token(_group)" and with scale_ue8m0=True),
    prepare("quant_static", x, scale, out=q),
    prepare("scaled_mm_channelwise", a, b, a_scale, b_scale, bias=None, out=out, config=None),
    prepare("scaled_mm_blockwise", a, b, a_scale, b_scale, bias=None, m=None, out=out,
    config=None), prepare("linear_channelwise", x, w_q, w_s, bias=None, out=out, q=q,
    scale=s, config=None), prepare("linear_blockwise", x, w_q, w_s, bias=None,
    row_alignment=4, out=out, q=q, scale=st, config=None) (st: [K/128, M_pad]
    storage): validate once (by running the op once) and return a Prepared."""
    lib = _lib.load()
    if op in ("linear_channelwise", "linear_blockwise"):
        kw = {k_: v for k_, v in kwargs.items() if k_ not in ("out", "q", "scale")}
        globals()[op](*args, **kw)  # validates and raises on bad arguments
    else:
        globals()[op](*args, **kwargs)
    if op in ("quant_per_token", "silu_mul_quant_per_token"):
        x = args[0]
        q, s = kwargs["out"], kwargs["scale"]
        silu = op == "silu_mul_quant_per_token"
        k = x.shape[1] // 2 if silu else x.shape[1]
        a = (_p(x), x.shape[0], k, x.stride(0), _p(q), q.stride(0), _p(s),
             ctypes.c_float(kwargs.get("eps", 1e-10)),
             _flags(silu or kwargs.get("silu_mul", False), kwargs.get("scale_ue8m0", False)),
             _stream(x))
        return Prepared(lib.fp8_quant_per_token_ex, a, op, (x, q, s))
    if op in ("quant_per_token_group", "silu_mul_quant_per_token_group"):
        x, g = args[0], args[1]
        q, st = kwargs["out"], kwargs["scale_storage"]
        silu = op == "silu_mul_quant_per_token_group" or kwargs.get("silu_mul", False)
        k = x.shape[1] // 2 if silu else x.shape[1]
        a = (_p(x), x.shape[0], k, x.stride(0), g, kwargs.get("row_alignment", 4), _p(q),
             q.stride(0), _p(st), ctypes.c_float(kwargs.get("eps", 1e-10)),
             _flags(silu, kwargs.get("scale_ue8m0", False)), _stream(x))
        return Prepared(lib.fp8_quant_per_token_group_ex, a, op, (x, q, st))
    if op == "quant_static":
        x, scale = args[0], args[1]
        q = kwargs["out"]
        a = (_p(x), x.shape[0], x.shape[1], x.stride(0), _p(scale), _p(q), q.stride(0), _stream(x))
        return Prepared(lib.fp8_quant_static, a, op, (x, scale, q))
    if op in ("linear_channelwise", "linear_blockwise"):
        kind = KIND_CHANNELWISE if op == "linear_channelwise" else KIND_BLOCKWISE
        x, w_q, w_s = args[0], args[1], args[2]
        cfg = kwargs.get("config") or TileConfig(-1, 0, 0, 0, 1, 0)
        a, keep = _linear_args(kind, x, w_q, w_s, kwargs.get("bias"), kwargs.get("eps", 1e-10),
                               kwargs.get("row_alignment", 4), cfg, kwargs["out"], kwargs["q"],
                               kwargs["scale"], _flags(kwargs.get("silu_mul", False),
                                                       kwargs.get("scale_ue8m0", False)))
        return Prepared(lib.fp8_linear_channelwise_ex if op == "linear_channelwise"
                        else lib.fp8_linear_blockwise_ex, a, op, keep + (x, w_q, w_s, kwargs.get("bias")))
    if op in ("scaled_mm_channelwise", "scaled_mm_blockwise"):
        a_, b_, sa, sb = _as_codes(args[0], "a"), _as_codes(args[1], "b"), args[2], args[3]
        bias, out = kwargs.get("bias"), kwargs["out"]
        cfg = kwargs.get("config") or TileConfig(-1, 0, 0, 0, 1, 0)
        n, k = b_.shape[0], a_.shape[1]
        if op == "scaled_mm_channelwise":
            m = a_.shape[0]
            nws = workspace_bytes(KIND_CHANNELWISE, m, n, k, cfg)
            ws = _ws.get(a_.device, nws)
            a = (_p(a_), _p(b_), _p(sa), _p(sb), _p(bias), _p(out), m, n, k, a_.stride(0),
                 b_.stride(0), out.stride(0), _p(ws), nws, ctypes.byref(cfg), _stream(a_))
            pr = Prepared(lib.fp8_scaled_mm_channelwise_ex, a, op, (a_, b_, sa, sb, bias, out, cfg, ws))
        else:
            m = kwargs.get("m") or a_.shape[0]
            nws = workspace_bytes(KIND_BLOCKWISE, m, n, k, cfg)
            ws = _ws.get(a_.device, nws)
            a = (_p(a_), _p(b_), _p(sa), sa.stride(1), _p(sb), _p(bias), _p(out), m, n, k,
                 a_.stride(0), b_.stride(0), out.stride(0), _p(ws), nws, ctypes.byref(cfg),
                 _stream(a_))
            fn = lib.fp8_scaled_mm_blockwise_ue8m0_ex if kwargs.get("scale_ue8m0") else \
                lib.fp8_scaled_mm_blockwise_ex
            pr = Prepared(fn, a, op, (a_, b_, sa, sb, bias, out, cfg, ws))
        return pr
    raise ValueError(f"unknown op {op}")
