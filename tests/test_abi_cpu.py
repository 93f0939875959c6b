"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/bsa.h declares, and rejects bad arguments with the documented
status before making any HIP call."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_build_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"BSA_API\s+[\w\s\*]+?\b(bsa_\w+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["bsa_build_block_desc", "bsa_select_blocks", "bsa_append_select",
              "bsa_sparse_decode", "bsa_sparse_decode_gated", "bsa_rectify_chunk",
              "bsa_workspace_size",
              "bsa_status_string", "bsa_block_count"]:
        assert n in names
    assert sorted(bsa.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    L = bsa.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_no_internal_symbols_exported():
    # only the C entry points are visible from the shared object
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", bsa._LIBPATH], capture_output=True,
                         text=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert {s for s in syms if s.startswith("bsa_")} == set(declared_functions())
    assert not any("launch_" in s for s in syms)


def test_status_strings():
    for s in range(8):
        assert bsa.status_string(s)
    assert "contract" in bsa.status_string(bsa.ERR_CONTRACT)
    assert bsa.status_string(99) == "unknown status"


@pytest.fixture
def checked_lib():
    before = bsa.use_library(bsa.LIB_CHECKED)
    try:
        yield bsa.lib()
    finally:
        bsa.use_library(before)


def test_checked_library_exports_the_same_symbols(checked_lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", bsa.LIB_CHECKED], capture_output=True,
                         text=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert {s for s in syms if s.startswith("bsa_")} == set(declared_functions())
    for n in declared_functions():
        assert hasattr(checked_lib, n), n


def test_checked_library_validates_host_arguments_first(checked_lib):
    # host-side validation still runs before any HIP call, so these statuses
    # come back without a device (the contract checks would need one)
    fake = ctypes.c_void_p(0x1000)
    C = bsa.c_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    for kw, status in [(dict(Hq=30), bsa.ERR_SHAPE), (dict(d=96), bsa.ERR_UNSUPPORTED)]:
        st = checked_lib.bsa_build_block_desc(ctypes.byref(L_ok(**kw).c()), ctypes.byref(C),
                                              fake, fake, 1, None, None)
        assert st == status
    P = bsa.SelectParams(sparsity_bp=9000, n_local=2, n_max=10)
    assert _select(L_ok(), P, q=0) == bsa.ERR_NULL
    assert _select(L_ok(), P, ws_bytes=16) == bsa.ERR_WORKSPACE
    assert _select(L_ok(), bsa.SelectParams(sparsity_bp=9000, n_local=0, n_max=10)) == bsa.ERR_PARAM


def L_ok(**kw):
    base = dict(B=2, Hq=32, Hkv=8, d=128, block=64, max_blocks=100,
                kv_dtype=bsa.DTYPE_BF16, desc_kind=bsa.DESC_MINMAX)
    base.update(kw)
    return bsa.Layout(**base)


def test_workspace_size():
    L = L_ok()
    assert bsa.workspace_size(L, bsa.OP_SELECT, 10) >= 2 * 8 * 100 * 4
    assert bsa.workspace_size(L, bsa.OP_DECODE, 10) > 2 * 32 * 128 * 4
    assert bsa.workspace_size(L, bsa.OP_RECTIFY, 32) > 2 * 32 * 32 * 128 * 4
    assert bsa.workspace_size(L, 99, 10) == 0
    assert bsa.workspace_size(L_ok(d=96), bsa.OP_DECODE, 10) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=30), bsa.ERR_SHAPE),
    (dict(B=0), bsa.ERR_SHAPE),
    (dict(d=96), bsa.ERR_UNSUPPORTED),
    (dict(block=48), bsa.ERR_UNSUPPORTED),
    (dict(kv_dtype=7), bsa.ERR_UNSUPPORTED),
    (dict(desc_kind=3), bsa.ERR_UNSUPPORTED),
    (dict(Hq=8 * 32), bsa.ERR_UNSUPPORTED),        # G = 32 > 16
    (dict(max_blocks=40000), bsa.ERR_UNSUPPORTED),
])
def test_layout_rejected_before_any_hip_call(kw, status):
    L = L_ok(**kw)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    C = bsa.c_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    st = bsa.lib().bsa_build_block_desc(ctypes.byref(L.c()), ctypes.byref(C), fake, fake, 1,
                                        None, None)
    assert st == status


def _select(L, P, ws_bytes=1 << 30, q=0x1000, cache_ptr=0x1000):
    C = bsa.c_cache(cache_ptr, 0x1000, 0x1000, 0x1000, 0x1000)
    p = ctypes.c_void_p(0x1000)
    return bsa.lib().bsa_select_blocks(ctypes.byref(L.c()), ctypes.byref(C),
                                       ctypes.c_void_p(q) if q else None,
                                       ctypes.byref(P.c()), p, p, p, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_local=0), bsa.ERR_PARAM),
    (dict(n_min=-1), bsa.ERR_PARAM),
    (dict(budget_tokens=-5), bsa.ERR_PARAM),
    (dict(sparsity_bp=10000), bsa.ERR_PARAM),
    (dict(sparsity_bp=-1), bsa.ERR_PARAM),
    (dict(n_max=5), bsa.ERR_PARAM),                 # needs 10 for NB = 100, p = 0.9
])
def test_select_params_rejected(kw, status):
    base = dict(sparsity_bp=9000, n_local=2, n_min=0, n_max=10)
    base.update(kw)
    assert _select(L_ok(), bsa.SelectParams(**base)) == status


def test_select_null_and_workspace():
    P = bsa.SelectParams(sparsity_bp=9000, n_local=2, n_max=10)
    assert _select(L_ok(), P, q=0) == bsa.ERR_NULL
    assert _select(L_ok(), P, cache_ptr=0) == bsa.ERR_NULL
    assert _select(L_ok(), P, ws_bytes=16) == bsa.ERR_WORKSPACE
    # mean-pool descriptors need a gate weight
    assert _select(L_ok(desc_kind=bsa.DESC_MEANPOOL), P) == bsa.ERR_PARAM


def test_append_select_validation():
    L = L_ok()
    C = bsa.c_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    p = ctypes.c_void_p(0x1000)
    lib = bsa.lib()
    P = bsa.SelectParams(sparsity_bp=9000, n_local=2, n_max=10)

    def call(L=L, k=p, v=p, P=P, ws_bytes=1 << 30):
        return lib.bsa_append_select(ctypes.byref(L.c()), ctypes.byref(C), k, v, p,
                                     ctypes.byref(P.c()), p, p, p, ws_bytes, None)
    assert call(k=None) == bsa.ERR_NULL
    assert call(v=None) == bsa.ERR_NULL
    assert call(P=bsa.SelectParams(sparsity_bp=9000, n_local=0, n_max=10)) == bsa.ERR_PARAM
    assert call(ws_bytes=16) == bsa.ERR_WORKSPACE
    assert call(L=L_ok(d=96)) == bsa.ERR_UNSUPPORTED


def test_append_select_decode_validation():
    L = L_ok()
    C = bsa.c_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    p = ctypes.c_void_p(0x1000)
    lib = bsa.lib()
    P = bsa.SelectParams(sparsity_bp=9000, n_local=2, n_max=10)
    need = bsa.workspace_size(L, bsa.OP_STEP, 10)
    # the step's workspace holds the scores, then the decode's partials
    assert need == (bsa.workspace_size(L, bsa.OP_SELECT, 10)
                    + bsa.workspace_size(L, bsa.OP_DECODE, 10))

    def call(L=L, k=p, v=p, P=P, o=p, scale=0.1, ws_bytes=need):
        return lib.bsa_append_select_decode(ctypes.byref(L.c()), ctypes.byref(C), k, v, p,
                                            ctypes.byref(P.c()), p, p, scale, o, p, p, ws_bytes,
                                            None)
    assert call(k=None) == bsa.ERR_NULL
    assert call(o=None) == bsa.ERR_NULL
    assert call(P=bsa.SelectParams(sparsity_bp=9000, n_local=0, n_max=10)) == bsa.ERR_PARAM
    assert call(P=bsa.SelectParams(sparsity_bp=9000, n_local=2, n_max=5)) == bsa.ERR_PARAM
    # n_max beyond the layout's capacity (the decode's bound)
    assert call(P=bsa.SelectParams(sparsity_bp=9000, n_local=2, n_max=101),
                ws_bytes=1 << 30) == bsa.ERR_PARAM
    assert call(scale=0.0) == bsa.ERR_PARAM
    assert call(scale=float("inf")) == bsa.ERR_PARAM
    assert call(ws_bytes=need - 1) == bsa.ERR_WORKSPACE
    assert call(L=L_ok(d=96)) == bsa.ERR_UNSUPPORTED


class _FakeDev:
    """Stands in for a device tensor in validation calls that never launch."""
    def data_ptr(self):
        return 0x1000


@pytest.mark.parametrize("tau", [-0.5, float("nan"), float("inf")])
def test_gate_tau_rejected_when_bias_requested(tau):
    P = bsa.SelectParams(sparsity_bp=9000, n_local=2, n_max=10, gate_tau=tau,
                         gate_bias=_FakeDev())
    assert _select(L_ok(), P) == bsa.ERR_PARAM
    assert bsa.block_count(P, 100, 64) == 10   # the count ignores the gate


@pytest.mark.parametrize("gc", [-1, 3])
def test_gate_current_rejected_outside_the_local_blocks(gc):
    # with a bias requested, the current blocks are 0 (= 1) .. n_local of the
    # local blocks; without one the field is not read
    P = bsa.SelectParams(sparsity_bp=9000, n_local=2, n_max=10, gate_tau=0.1,
                         gate_bias=_FakeDev(), gate_current=gc)
    assert _select(L_ok(), P) == bsa.ERR_PARAM
    P2 = bsa.SelectParams(sparsity_bp=9000, n_local=2, n_max=10, gate_current=gc)
    assert _select(L_ok(), P2, ws_bytes=16) == bsa.ERR_WORKSPACE  # validation went past it


def test_decode_gated_validation():
    L = L_ok()
    C = bsa.c_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    p = ctypes.c_void_p(0x1000)
    lib = bsa.lib()

    def call(bias=p, scale=0.1, ws_bytes=1 << 30, idx=p):
        return lib.bsa_sparse_decode_gated(ctypes.byref(L.c()), ctypes.byref(C), p, idx, p, bias,
                                           10, scale, p, p, p, ws_bytes, None)
    assert call(bias=None) == bsa.ERR_NULL
    assert call(idx=None) == bsa.ERR_NULL
    assert call(scale=-1.0) == bsa.ERR_PARAM
    assert call(ws_bytes=64) == bsa.ERR_WORKSPACE


def test_decode_and_rectify_validation():
    L = L_ok()
    C = bsa.c_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    p = ctypes.c_void_p(0x1000)
    lib = bsa.lib()
    st = lib.bsa_sparse_decode(ctypes.byref(L.c()), ctypes.byref(C), p, p, p, 10, 0.0, p, p, p,
                               1 << 30, None)
    assert st == bsa.ERR_PARAM  # scale must be > 0
    st = lib.bsa_sparse_decode(ctypes.byref(L.c()), ctypes.byref(C), p, p, p, 10, float("nan"),
                               p, p, p, 1 << 30, None)
    assert st == bsa.ERR_PARAM
    st = lib.bsa_sparse_decode(ctypes.byref(L.c()), ctypes.byref(C), p, p, p, 10, 0.1, p, p, p,
                               64, None)
    assert st == bsa.ERR_WORKSPACE
    st = lib.bsa_sparse_decode(ctypes.byref(L.c()), ctypes.byref(C), p, None, p, 10, 0.1, p, p,
                               p, 1 << 30, None)
    assert st == bsa.ERR_NULL
    st = lib.bsa_rectify_chunk(ctypes.byref(L.c()), ctypes.byref(C), p, p, p, 0, 0.1, p, p, p,
                               1 << 30, None)
    assert st == bsa.ERR_PARAM
    st = lib.bsa_rectify_chunk(ctypes.byref(L.c()), ctypes.byref(C), p, p, p, 32, 0.1, p, p, p,
                               1024, None)
    assert st == bsa.ERR_WORKSPACE
    st = lib.bsa_rectify_chunk(ctypes.byref(L.c()), ctypes.byref(C), p, p, p, 32 * 100 * 64,
                               0.1, p, p, p, 1 << 40, None)
    assert st == bsa.ERR_PARAM   # f beyond the capacity


def test_build_block_desc_argument_rules():
    L = L_ok()
    C = bsa.c_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    p = ctypes.c_void_p(0x1000)
    lib = bsa.lib()
    assert lib.bsa_build_block_desc(ctypes.byref(L.c()), ctypes.byref(C), p, None, 1, None,
                                    None) == bsa.ERR_PARAM
    assert lib.bsa_build_block_desc(ctypes.byref(L.c()), ctypes.byref(C), p, p, 0, None,
                                    None) == bsa.ERR_PARAM
    assert lib.bsa_build_block_desc(ctypes.byref(L.c()), ctypes.byref(C), p, p, 1, p,
                                    None) == bsa.ERR_PARAM
    assert lib.bsa_build_block_desc(None, ctypes.byref(C), p, p, 1, None, None) == bsa.ERR_NULL


def test_host_block_count_matches_oracle():
    import oracle as O
    for budget, bp, nl, nm in [(512, 0, 1, 2), (4096, 0, 1, 0), (0, 9000, 2, 16),
                               (0, 9500, 2, 16), (0, 9800, 2, 0), (0, 0, 1, 0)]:
        P = bsa.SelectParams(budget_tokens=budget, sparsity_bp=bp, n_local=nl, n_min=nm)
        for NB in [1, 2, 5, 33, 257, 513, 2049, 8193]:
            assert bsa.block_count(P, NB, 64) == O.block_count(NB, 64, budget, bp, nl, nm)


def test_binding_refuses_host_tensors_and_non_tensors():
    """The Python wrappers hand the library data pointers only, so they check
    every tensor first: a host tensor or a non-tensor is refused before any
    library call (the GPU-side dtype, layout and size checks are in
    tests/test_gpu_binding.py)."""
    import torch
    L = bsa.Layout(1, 4, 1, 64, 64, 4, bsa.DTYPE_F32, bsa.DESC_MINMAX)
    C = bsa.Cache(torch.zeros(4, 1, 64 * 64), torch.zeros(4, 1, 64 * 64),
                  torch.zeros(1, 4, dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                  torch.zeros(1, 1, 4, 2, 64))
    q = torch.zeros(1, 4, 64)
    idx = torch.zeros(1, 1, 2, dtype=torch.int32)
    cnt = torch.zeros(1, 1, dtype=torch.int32)
    o, lse, ws = torch.zeros(1, 4, 64), torch.zeros(1, 4), torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        bsa.sparse_decode(L, C, q, idx, cnt, 2, 0.125, o, lse, ws)
    P = bsa.SelectParams(budget_tokens=128, n_local=1, n_max=2)
    with pytest.raises(ValueError, match="GPU tensor"):
        bsa.select_blocks(L, C, q, P, idx, cnt, ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        bsa.build_block_desc(L, C)
    with pytest.raises(ValueError, match="GPU tensor"):
        bsa.rectify_chunk(L, C, q, q, q, 1, 0.125, o, lse, ws)
    C_list = bsa.Cache([0.0], C.v_pool, C.page_table, C.seq_lens, C.desc)
    with pytest.raises(TypeError, match="torch tensor"):
        bsa.sparse_decode(L, C_list, q, idx, cnt, 2, 0.125, o, lse, ws)


def test_static_scratch_decode_validates_before_any_hip_call():
    # the decode without a workspace refuses a call whose split partials
    # exceed the library's scratch array, and bad arguments, on the host
    fake = ctypes.c_void_p(0x1000)
    C = bsa.c_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    big = L_ok(B=256, Hq=128, Hkv=8, max_blocks=64)
    assert bsa.workspace_size(big, bsa.OP_DECODE, 16) > bsa.STATIC_SCRATCH_BYTES
    f = bsa.lib().bsa_sparse_decode_static
    assert f(ctypes.byref(big.c()), ctypes.byref(C), fake, fake, fake, 16, 0.1, fake, fake,
             None) == bsa.ERR_WORKSPACE
    L = L_ok()
    assert f(ctypes.byref(L.c()), ctypes.byref(C), None, fake, fake, 10, 0.1, fake, fake,
             None) == bsa.ERR_NULL
    assert f(ctypes.byref(L.c()), ctypes.byref(C), fake, fake, fake, 0, 0.1, fake, fake,
             None) == bsa.ERR_PARAM
    assert f(ctypes.byref(L.c()), ctypes.byref(C), fake, fake, fake, 10, -1.0, fake, fake,
             None) == bsa.ERR_PARAM
    assert f(ctypes.byref(L_ok(d=96).c()), ctypes.byref(C), fake, fake, fake, 10, 0.1, fake,
             fake, None) == bsa.ERR_UNSUPPORTED


def test_read_probe_rejects_bad_arguments_before_any_launch():
    """The benchmark's read probe (libbsa_probe.so, outside the interface):
    its two exports load, and arguments it cannot serve return -1 before any
    HIP call (a null buffer or sink, no workgroups, a size that is not whole
    16-byte loads, an unknown mode, and for the scattered-chunk mode a size
    that is not whole 16 KiB chunks)."""
    path = os.path.join(ROOT, "block_sparse_attention_build_amd", "libbsa_probe.so")
    P = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    P.bsa_probe_read_mode.argtypes = [vp, sz, vp, i32, i32, vp]
    P.bsa_probe_read_mode.restype = i32
    P.bsa_probe_read.argtypes = [vp, sz, vp, i32, vp]
    P.bsa_probe_read.restype = i32
    fake = ctypes.c_void_p(0x1000)
    assert P.bsa_probe_read(None, 1 << 20, fake, 8, None) == -1
    assert P.bsa_probe_read(fake, 1 << 20, None, 8, None) == -1
    assert P.bsa_probe_read(fake, 1 << 20, fake, 0, None) == -1
    assert P.bsa_probe_read(fake, (1 << 20) + 8, fake, 8, None) == -1
    for mode in (-1, 4):
        assert P.bsa_probe_read_mode(fake, 1 << 20, fake, 8, mode, None) == -1
    assert P.bsa_probe_read_mode(fake, (16 << 10) + 16, fake, 8, 3, None) == -1
    assert P.bsa_probe_read_mode(fake, 0, fake, 8, 3, None) == -1
