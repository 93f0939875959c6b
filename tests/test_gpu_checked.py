"""The checked build (libbsa_checked.so).

On valid inputs it gives exactly the default library's results (the same
kernels run after the host-side checks).  For each device-side contract the
header lists it returns BSA_ERR_CONTRACT before enqueuing anything, so the
outputs stay untouched.  The broken inputs below are also chosen so that
every access a kernel would make with them stays inside the allocations:
over-long sequences sit at s = 0 of a two-sequence batch (their extra block
indexes the next row of the page table), out-of-range block ids index a row
that exists, and no page id 0 sits where a negative position would land."""
import math

import numpy as np
import pytest

import block_sparse_attention_build_amd as bsa
import workloads as W
from harness import prefill, to_dev

pytestmark = pytest.mark.gpu

BF16, MINMAX = bsa.DTYPE_BF16, bsa.DESC_MINMAX
B, HQ, HKV, D, BLK, MAXB = 2, 8, 2, 64, 64, 16
LENGTHS = [700, 300]
F = 32


def _torch():
    import torch
    return torch


@pytest.fixture
def checked():
    before = bsa.use_library(bsa.LIB_CHECKED)
    try:
        yield
    finally:
        bsa.use_library(before)


class State:
    """A small cache, a query, a selection and outputs, on the library in
    use when it is built."""

    def __init__(self, seed=41):
        torch = _torch()
        self.L = bsa.Layout(B, HQ, HKV, D, BLK, MAXB, BF16, MINMAX)
        rng = np.random.Generator(np.random.PCG64(seed))
        self.Ks = [W.quantize(rng.standard_normal((HKV, T, D), dtype=np.float32), "bf16")
                   for T in LENGTHS]
        self.Vs = [W.quantize(rng.standard_normal((HKV, T, D), dtype=np.float32), "bf16")
                   for T in LENGTHS]
        q = W.quantize(rng.standard_normal((B, HQ, D), dtype=np.float32), "bf16")
        self.qr = to_dev(W.quantize(rng.standard_normal((B, HQ, F, D), dtype=np.float32), "bf16"),
                         self.L)
        self.kr = to_dev(W.quantize(rng.standard_normal((B, HKV, F, D), dtype=np.float32), "bf16"),
                         self.L)
        self.vr = to_dev(W.quantize(rng.standard_normal((B, HKV, F, D), dtype=np.float32), "bf16"),
                         self.L)
        # pages in reverse order: no sequence starts at page 0
        pt = torch.arange(B * MAXB, dtype=torch.int32).flip(0).reshape(B, MAXB).contiguous()
        self.cache = bsa.allocate_cache(self.L, page_table=pt)
        for t in (self.cache.k_pool, self.cache.v_pool, self.cache.desc):
            t.zero_()  # unused pages compare equal between two states
        prefill(self.L, self.cache, self.Ks, self.Vs, LENGTHS)
        self.q = to_dev(q, self.L)
        self.P = bsa.SelectParams(sparsity_bp=7000, n_local=1, n_min=2)
        self.P.n_max = bsa.block_count(self.P, MAXB, BLK)
        self.idx = torch.full((B, HKV, self.P.n_max), -7, dtype=torch.int32, device="cuda")
        self.cnt = torch.full((B, HKV), -7, dtype=torch.int32, device="cuda")
        self.bias = torch.zeros(B, HKV, self.P.n_max, dtype=torch.float32, device="cuda")
        n = max(bsa.workspace_size(self.L, op, a) for op, a in
                [(bsa.OP_SELECT, self.P.n_max), (bsa.OP_DECODE, self.P.n_max),
                 (bsa.OP_RECTIFY, F)])
        self.ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        self.fresh_outputs()

    def fresh_outputs(self):
        torch = _torch()
        self.o = torch.full((B, HQ, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.full((B, HQ), float("nan"), dtype=torch.float32, device="cuda")
        self.o_r = torch.full((B, HQ, F, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.lse_r = torch.full((B, HQ, F), float("nan"), dtype=torch.float32, device="cuda")

    def select(self):
        bsa.select_blocks(self.L, self.cache, self.q, self.P, self.idx, self.cnt, self.ws)

    def decode(self, gated=False):
        if gated:
            bsa.sparse_decode_gated(self.L, self.cache, self.q, self.idx, self.cnt, self.bias,
                                    self.P.n_max, 1 / math.sqrt(D), self.o, self.lse, self.ws)
        else:
            bsa.sparse_decode(self.L, self.cache, self.q, self.idx, self.cnt, self.P.n_max,
                              1 / math.sqrt(D), self.o, self.lse, self.ws)

    def rectify(self):
        bsa.rectify_chunk(self.L, self.cache, self.qr, self.kr, self.vr, F, 1 / math.sqrt(D),
                          self.o_r, self.lse_r, self.ws)

    def step(self):
        """select, plain and gated decode, rectify, then an append + select."""
        torch = _torch()
        self.P.gate_tau, self.P.gate_bias = 0.02, self.bias
        self.select()
        self.decode()
        out = [self.idx.clone(), self.cnt.clone(), self.bias.clone(), self.o.clone(),
               self.lse.clone()]
        self.decode(gated=True)
        out += [self.o.clone(), self.lse.clone()]
        self.rectify()
        out += [self.o_r.clone(), self.lse_r.clone()]
        self.cache.seq_lens += 1
        kn = torch.ones(B, HKV, 1, D, dtype=torch.bfloat16, device="cuda")
        bsa.append_select(self.L, self.cache, kn, -kn, self.q, self.P, self.idx, self.cnt,
                          self.ws)
        out += [self.idx.clone(), self.cnt.clone(), self.cache.k_pool.clone(),
                self.cache.v_pool.clone(), self.cache.desc.clone()]
        torch.cuda.synchronize()
        return out


def test_checked_build_equals_the_default_build():
    torch = _torch()
    ref = State().step()
    before = bsa.use_library(bsa.LIB_CHECKED)
    try:
        got = State().step()
    finally:
        bsa.use_library(before)
    assert len(ref) == len(got) == 14
    for i, (a, b) in enumerate(zip(ref, got)):
        # bit patterns: the same kernels on the same inputs
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), i


def _rejected(fn):
    with pytest.raises(bsa.BsaError) as e:
        fn()
    assert e.value.status == bsa.ERR_CONTRACT, e.value


def _untouched(S):
    torch = _torch()
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(S.o.float())) and torch.all(torch.isnan(S.lse))
    assert torch.all(torch.isnan(S.o_r.float())) and torch.all(torch.isnan(S.lse_r))


def test_lengths_beyond_capacity_are_rejected(checked):
    torch = _torch()
    S = State()
    S.select()
    torch.cuda.synchronize()
    idx0 = S.idx.clone()
    S.cache.seq_lens[0] = MAXB * BLK + 1
    _rejected(S.select)
    _rejected(S.decode)
    _rejected(S.rectify)
    _rejected(lambda: bsa.build_block_desc(S.L, S.cache))  # rebuild mode
    kn = torch.zeros(B, HKV, 1, D, dtype=torch.bfloat16, device="cuda")
    _rejected(lambda: bsa.append_select(S.L, S.cache, kn, kn, S.q, S.P, S.idx, S.cnt, S.ws))
    _untouched(S)
    assert torch.equal(S.idx, idx0)
    # the same state with its length restored runs
    S.cache.seq_lens[0] = LENGTHS[0]
    S.select()
    torch.cuda.synchronize()
    assert torch.equal(S.idx, idx0)


def test_append_and_rectify_longer_than_the_sequence_are_rejected(checked):
    torch = _torch()
    S = State()
    kn = torch.zeros(B, HKV, 1, D, dtype=torch.bfloat16, device="cuda")
    S.cache.seq_lens[1] = 0
    _rejected(lambda: bsa.build_block_desc(S.L, S.cache, kn, kn, 1))
    _rejected(lambda: bsa.append_select(S.L, S.cache, kn, kn, S.q, S.P, S.idx, S.cnt, S.ws))
    S.cache.seq_lens[1] = F - 1
    _rejected(S.rectify)
    _untouched(S)
    assert torch.all(S.idx == -7)


def test_negative_page_id_is_rejected(checked):
    S = State()
    S.cache.page_table[0, 3] = -1  # block 3 of sequence 0 holds tokens
    _rejected(S.select)
    assert bool((S.idx == -7).all())
    S.cache.page_table[0, 15] = -1  # past the tokens: not a contract
    S.cache.page_table[0, 3] = B * MAXB - 1 - 3  # its own page again
    S.select()


@pytest.mark.parametrize("case", ["cnt_above_n_max", "cnt_negative", "id_repeated",
                                  "id_past_the_sequence", "id_negative", "bias_inf",
                                  "bias_nan"])
def test_broken_kept_lists_are_rejected(checked, case):
    torch = _torch()
    S = State()
    S.P.gate_tau, S.P.gate_bias = 0.02, S.bias
    S.select()
    torch.cuda.synchronize()
    gated = case.startswith("bias")
    c = int(S.cnt[1, 0])
    assert c >= 2
    if case == "cnt_above_n_max":
        S.cnt[0, 0] = S.P.n_max + 1
    elif case == "cnt_negative":
        S.cnt[1, 1] = -1
    elif case == "id_repeated":
        S.idx[1, 0, 1] = S.idx[1, 0, 0]
    elif case == "id_past_the_sequence":
        S.idx[1, 0, c - 1] = (LENGTHS[1] + BLK - 1) // BLK  # first block past T
    elif case == "id_negative":
        S.idx[1, 0, 0] = -1
    elif case == "bias_inf":
        S.bias[1, 0, c - 1] = float("inf")
    else:
        S.bias[0, 1, 0] = float("nan")
    _rejected(lambda: S.decode(gated=gated))
    _untouched(S)
    # entries past cnt are not part of the contract
    S2 = State()
    S2.select()
    torch.cuda.synchronize()
    if S2.cnt[1, 0] < S2.P.n_max:
        S2.idx[1, 0, -1] = 12345
    S2.decode()
    torch.cuda.synchronize()
    assert not torch.any(torch.isnan(S2.lse))
