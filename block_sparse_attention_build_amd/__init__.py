"""Python binding of libbsa (block-sparse attention decoding on MI355X).

A thin ctypes layer over the C ABI in include/bsa.h: the functions below have
the C entry points' names and arguments, take torch tensors that live on the
GPU, check that each is a contiguous GPU tensor of the documented dtype and
at least the documented size, and pass their data pointers and the current
HIP stream.  torch supplies device memory and streams only; every step of
the computation runs in the library's HIP kernels.  There is no CPU
fallback: if libbsa.so is missing or fails to load, every call raises.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_DEFAULT = os.path.join(_PKG, "libbsa.so")
# the build that verifies device-side contracts on the host (synchronises)
LIB_CHECKED = os.path.join(_PKG, "libbsa_checked.so")
_LIBPATH = LIB_CHECKED if os.environ.get("BSA_CHECKED") == "1" else LIB_DEFAULT

# status codes (bsa_status)
(OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_PARAM, ERR_WORKSPACE, ERR_HIP,
 ERR_CONTRACT) = range(8)
DTYPE_F32, DTYPE_BF16 = 0, 1
DESC_MINMAX, DESC_MEANPOOL = 0, 1
OP_SELECT, OP_DECODE, OP_RECTIFY, OP_STEP = 1, 2, 3, 4

EXPORTS = ("bsa_build_block_desc", "bsa_select_blocks", "bsa_append_select",
           "bsa_append_select_decode", "bsa_sparse_decode", "bsa_sparse_decode_gated", "bsa_sparse_decode_static",
           "bsa_rectify_chunk", "bsa_workspace_size", "bsa_block_count", "bsa_status_string")
# bytes of the library's per-GPU scratch array (bsa_sparse_decode_static)
STATIC_SCRATCH_BYTES = 16 << 20


class BsaError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class c_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "Hq", "Hkv", "d", "block", "max_blocks", "kv_dtype", "desc_kind")]


class c_cache(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("desc", ctypes.c_void_p)]


class c_select_params(ctypes.Structure):
    _fields_ = [("budget_tokens", ctypes.c_int32), ("sparsity_bp", ctypes.c_int32),
                ("n_local", ctypes.c_int32), ("n_min", ctypes.c_int32),
                ("n_max", ctypes.c_int32), ("gate_w", ctypes.c_void_p),
                ("gate_tau", ctypes.c_float), ("gate_bias", ctypes.c_void_p),
                ("gate_current", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libbsa.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIBPATH):
        raise RuntimeError(f"{os.path.basename(_LIBPATH)} not found at {_LIBPATH}: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(_LIBPATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pl, pc, pp = ctypes.POINTER(c_layout), ctypes.POINTER(c_cache), ctypes.POINTER(c_select_params)
    L.bsa_build_block_desc.argtypes = [pl, pc, vp, vp, i32, vp, vp]
    L.bsa_select_blocks.argtypes = [pl, pc, vp, pp, vp, vp, vp, sz, vp]
    L.bsa_append_select.argtypes = [pl, pc, vp, vp, vp, pp, vp, vp, vp, sz, vp]
    L.bsa_append_select_decode.argtypes = [pl, pc, vp, vp, vp, pp, vp, vp, ctypes.c_float, vp,
                                           vp, vp, sz, vp]
    L.bsa_sparse_decode.argtypes = [pl, pc, vp, vp, vp, i32, ctypes.c_float, vp, vp, vp, sz, vp]
    L.bsa_sparse_decode_gated.argtypes = [pl, pc, vp, vp, vp, vp, i32, ctypes.c_float, vp, vp,
                                          vp, sz, vp]
    L.bsa_sparse_decode_static.argtypes = [pl, pc, vp, vp, vp, i32, ctypes.c_float, vp, vp, vp]
    L.bsa_rectify_chunk.argtypes = [pl, pc, vp, vp, vp, i32, ctypes.c_float, vp, vp, vp, sz, vp]
    L.bsa_workspace_size.argtypes = [pl, i32, i32]
    L.bsa_workspace_size.restype = sz
    L.bsa_block_count.argtypes = [pp, i32, i32]
    L.bsa_block_count.restype = i32
    L.bsa_status_string.argtypes = [ctypes.c_int]
    L.bsa_status_string.restype = ctypes.c_char_p
    for fn in (L.bsa_build_block_desc, L.bsa_select_blocks, L.bsa_append_select,
               L.bsa_append_select_decode, L.bsa_sparse_decode, L.bsa_sparse_decode_gated, L.bsa_sparse_decode_static,
               L.bsa_rectify_chunk):
        fn.restype = ctypes.c_int
    _lib = L
    return L


def use_library(path):
    """Switch every binding to the library at path (LIB_DEFAULT or
    LIB_CHECKED); returns the path in use before."""
    global _lib, _LIBPATH
    before = _LIBPATH
    _lib, _LIBPATH = None, path
    lib()
    return before


def status_string(status):
    return lib().bsa_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, what):
    if status != OK:
        raise BsaError(status, what)


def _need(t, name, dtype, numel):
    """t must be a contiguous GPU tensor of `dtype` (None: any) with at least
    `numel` elements: the library reaches it through its data pointer alone,
    so a wrong tensor is refused here rather than read out of bounds."""
    try:  # the common case in one expression: a few attribute reads per call
        if (t.is_cuda and (dtype is None or t.dtype == dtype) and t.is_contiguous()
                and t.numel() >= numel):
            return
    except AttributeError:
        pass
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor, got one on {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, needs at least {numel}")


def _need_cache(L, cache):
    import torch
    kv = L.torch_dtype()
    _need(cache.k_pool, "k_pool", kv, L.Hkv * L.block * L.d)
    _need(cache.v_pool, "v_pool", kv, L.Hkv * L.block * L.d)
    _need(cache.page_table, "page_table", torch.int32, L.B * L.max_blocks)
    _need(cache.seq_lens, "seq_lens", torch.int32, L.B)
    if L.desc_kind == DESC_MINMAX:
        _need(cache.desc, "desc", kv, L.B * L.Hkv * L.max_blocks * 2 * L.d)
    else:
        _need(cache.desc, "desc", torch.float32, L.B * L.Hkv * L.max_blocks * L.d)


def _need_select(L, cache, q, params, idx, cnt, ws):
    import torch
    _need_cache(L, cache)
    _need(q, "q", L.torch_dtype(), L.B * L.Hq * L.d)
    _need(idx, "idx", torch.int32, L.B * L.Hkv * params.n_max)
    _need(cnt, "cnt", torch.int32, L.B * L.Hkv)
    _need(ws, "ws", None, 0)
    if params.gate_w is not None:
        _need(params.gate_w, "gate_w", torch.bfloat16, L.d * L.d)
    if params.gate_bias is not None:
        _need(params.gate_bias, "gate_bias", torch.float32, L.B * L.Hkv * params.n_max)


def _need_decode(L, cache, q, idx, cnt, n_max, o, lse, ws):
    import torch
    _need_cache(L, cache)
    _need(q, "q", L.torch_dtype(), L.B * L.Hq * L.d)
    _need(idx, "idx", torch.int32, L.B * L.Hkv * n_max)
    _need(cnt, "cnt", torch.int32, L.B * L.Hkv)
    _need(o, "o", L.torch_dtype(), L.B * L.Hq * L.d)
    _need(lse, "lse", torch.float32, L.B * L.Hq)
    if ws is not None:
        _need(ws, "ws", None, 0)


# ---------------------------------------------------------------------------
# Shape / parameter records
# ---------------------------------------------------------------------------

@dataclass
class Layout:
    B: int
    Hq: int
    Hkv: int
    d: int
    block: int
    max_blocks: int
    kv_dtype: int = DTYPE_BF16
    desc_kind: int = DESC_MINMAX

    def c(self):
        return c_layout(self.B, self.Hq, self.Hkv, self.d, self.block, self.max_blocks,
                        self.kv_dtype, self.desc_kind)

    @property
    def G(self):
        return self.Hq // self.Hkv

    def torch_dtype(self):
        import torch
        return torch.bfloat16 if self.kv_dtype == DTYPE_BF16 else torch.float32


@dataclass
class SelectParams:
    budget_tokens: int = 0
    sparsity_bp: int = 0
    n_local: int = 1
    n_min: int = 0
    n_max: int = 0
    gate_w: Optional[object] = None  # torch bf16 [d, d] on the device
    gate_tau: float = 0.0
    gate_bias: Optional[object] = None  # torch fp32 [B, Hkv, n_max] on the device, OUT
    gate_current: int = 1  # trailing blocks with the unit gate (the page's current block: 1)

    def c(self):
        return c_select_params(self.budget_tokens, self.sparsity_bp, self.n_local, self.n_min,
                               self.n_max, None if self.gate_w is None else self.gate_w.data_ptr(),
                               float(self.gate_tau),
                               None if self.gate_bias is None else self.gate_bias.data_ptr(),
                               int(self.gate_current))


@dataclass
class Cache:
    """Device tensors of one paged cache (any torch tensors of the documented
    shapes; see PagedCache for an allocator)."""
    k_pool: object
    v_pool: object
    page_table: object
    seq_lens: object
    desc: object

    def c(self):
        return c_cache(self.k_pool.data_ptr(), self.v_pool.data_ptr(), self.page_table.data_ptr(),
                       self.seq_lens.data_ptr(), self.desc.data_ptr())


def allocate_cache(layout: Layout, num_pages: Optional[int] = None, page_table=None,
                   device="cuda"):
    """Allocate pools, descriptors and seq_lens with torch (device memory
    only).  page_table defaults to sequence s owning pages
    [s*max_blocks, (s+1)*max_blocks) in order."""
    import torch
    L = layout
    if num_pages is None:
        num_pages = L.B * L.max_blocks
    dt = L.torch_dtype()
    page_elems = L.block * L.d
    k_pool = torch.empty(num_pages, L.Hkv, page_elems, dtype=dt, device=device)
    v_pool = torch.empty(num_pages, L.Hkv, page_elems, dtype=dt, device=device)
    if page_table is None:
        page_table = torch.arange(L.B * L.max_blocks, dtype=torch.int32,
                                  device=device).view(L.B, L.max_blocks)
    else:
        page_table = page_table.to(device=device, dtype=torch.int32).contiguous()
    if L.desc_kind == DESC_MINMAX:
        desc = torch.empty(L.B, L.Hkv, L.max_blocks, 2, L.d, dtype=dt, device=device)
    else:
        desc = torch.empty(L.B, L.Hkv, L.max_blocks, L.d, dtype=torch.float32, device=device)
    seq_lens = torch.zeros(L.B, dtype=torch.int32, device=device)
    return Cache(k_pool, v_pool, page_table, seq_lens, desc)


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI, without the prefix)
# ---------------------------------------------------------------------------

def workspace_size(layout: Layout, op: int, n_max_or_f: int) -> int:
    return int(lib().bsa_workspace_size(ctypes.byref(layout.c()), op, n_max_or_f))


def block_count(params: SelectParams, NB: int, block: int) -> int:
    return int(lib().bsa_block_count(ctypes.byref(params.c()), NB, block))


def build_block_desc(layout: Layout, cache: Cache, k_new=None, v_new=None, n_new: int = 0,
                     range_begin=None, stream=None):
    """Append n_new tokens per sequence (k_new/v_new [B, Hkv, n_new, d]) or,
    with k_new = v_new = None, rebuild descriptors from range_begin [B]."""
    import torch
    _need_cache(layout, cache)
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        if t is not None:
            _need(t, name, layout.torch_dtype(), layout.B * layout.Hkv * int(n_new) * layout.d)
    if range_begin is not None:
        _need(range_begin, "range_begin", torch.int32, layout.B)
    st = lib().bsa_build_block_desc(ctypes.byref(layout.c()), ctypes.byref(cache.c()),
                                    _ptr(k_new), _ptr(v_new), int(n_new), _ptr(range_begin),
                                    _stream(stream))
    _check(st, "bsa_build_block_desc")


def select_blocks(layout: Layout, cache: Cache, q, params: SelectParams, idx, cnt, ws,
                  stream=None):
    _need_select(layout, cache, q, params, idx, cnt, ws)
    st = lib().bsa_select_blocks(ctypes.byref(layout.c()), ctypes.byref(cache.c()), _ptr(q),
                                 ctypes.byref(params.c()), _ptr(idx), _ptr(cnt), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "bsa_select_blocks")


def append_select(layout: Layout, cache: Cache, k_new, v_new, q, params: SelectParams, idx, cnt,
                  ws, stream=None):
    """build_block_desc (one token per sequence, k_new/v_new [B, Hkv, 1, d])
    followed by select_blocks, with the append sharing the scoring launch."""
    _need_select(layout, cache, q, params, idx, cnt, ws)
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, name, layout.torch_dtype(), layout.B * layout.Hkv * layout.d)
    st = lib().bsa_append_select(ctypes.byref(layout.c()), ctypes.byref(cache.c()), _ptr(k_new),
                                 _ptr(v_new), _ptr(q), ctypes.byref(params.c()), _ptr(idx),
                                 _ptr(cnt), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream))
    _check(st, "bsa_append_select")


def append_select_decode(layout: Layout, cache: Cache, k_new, v_new, q, params: SelectParams,
                         idx, cnt, softmax_scale: float, o, lse, ws, stream=None):
    """One decode step: append_select then sparse_decode (sparse_decode_gated
    when params.gate_bias is set), with the same results; ws holds at least
    workspace_size(layout, OP_STEP, params.n_max) bytes."""
    import torch
    L = layout
    _need_select(L, cache, q, params, idx, cnt, ws)
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, name, L.torch_dtype(), L.B * L.Hkv * L.d)
    _need(o, "o", L.torch_dtype(), L.B * L.Hq * L.d)
    _need(lse, "lse", torch.float32, L.B * L.Hq)
    st = lib().bsa_append_select_decode(ctypes.byref(L.c()), ctypes.byref(cache.c()), _ptr(k_new),
                                        _ptr(v_new), _ptr(q), ctypes.byref(params.c()), _ptr(idx),
                                        _ptr(cnt), float(softmax_scale), _ptr(o), _ptr(lse),
                                        _ptr(ws), ws.numel() * ws.element_size(),
                                        _stream(stream))
    _check(st, "bsa_append_select_decode")


def sparse_decode(layout: Layout, cache: Cache, q, idx, cnt, n_max: int, softmax_scale: float,
                  o, lse, ws, stream=None):
    _need_decode(layout, cache, q, idx, cnt, n_max, o, lse, ws)
    st = lib().bsa_sparse_decode(ctypes.byref(layout.c()), ctypes.byref(cache.c()), _ptr(q),
                                 _ptr(idx), _ptr(cnt), int(n_max), float(softmax_scale), _ptr(o),
                                 _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream))
    _check(st, "bsa_sparse_decode")


def sparse_decode_gated(layout: Layout, cache: Cache, q, idx, cnt, gate_bias, n_max: int,
                        softmax_scale: float, o, lse, ws, stream=None):
    """sparse_decode with gate_bias [B, Hkv, n_max] (fp32) added to the
    logits of every token of block idx[..., k]."""
    import torch
    _need_decode(layout, cache, q, idx, cnt, n_max, o, lse, ws)
    _need(gate_bias, "gate_bias", torch.float32, layout.B * layout.Hkv * n_max)
    st = lib().bsa_sparse_decode_gated(ctypes.byref(layout.c()), ctypes.byref(cache.c()),
                                       _ptr(q), _ptr(idx), _ptr(cnt), _ptr(gate_bias), int(n_max),
                                       float(softmax_scale), _ptr(o), _ptr(lse), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "bsa_sparse_decode_gated")


def sparse_decode_static(layout: Layout, cache: Cache, q, idx, cnt, n_max: int,
                         softmax_scale: float, o, lse, stream=None):
    """sparse_decode with the split partials in the library's per-GPU
    scratch array instead of a caller workspace (no allocation anywhere;
    calls that overlap on one GPU race)."""
    _need_decode(layout, cache, q, idx, cnt, n_max, o, lse, None)
    st = lib().bsa_sparse_decode_static(ctypes.byref(layout.c()), ctypes.byref(cache.c()),
                                        _ptr(q), _ptr(idx), _ptr(cnt), int(n_max),
                                        float(softmax_scale), _ptr(o), _ptr(lse), _stream(stream))
    _check(st, "bsa_sparse_decode_static")


def rectify_chunk(layout: Layout, cache: Cache, q, k_new, v_new, f: int, softmax_scale: float,
                  o, lse, ws, stream=None):
    import torch
    L, kv = layout, layout.torch_dtype()
    _need_cache(L, cache)
    _need(q, "q", kv, L.B * L.Hq * int(f) * L.d)
    _need(k_new, "k_new", kv, L.B * L.Hkv * int(f) * L.d)
    _need(v_new, "v_new", kv, L.B * L.Hkv * int(f) * L.d)
    _need(o, "o", kv, L.B * L.Hq * int(f) * L.d)
    _need(lse, "lse", torch.float32, L.B * L.Hq * int(f))
    _need(ws, "ws", None, 0)
    st = lib().bsa_rectify_chunk(ctypes.byref(layout.c()), ctypes.byref(cache.c()), _ptr(q),
                                 _ptr(k_new), _ptr(v_new), int(f), float(softmax_scale),
                                 _ptr(o), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream))
    _check(st, "bsa_rectify_chunk")
