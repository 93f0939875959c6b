"""Select + decode (plain and with the log-gate bias), and rectify, against
the oracle on seeded random shapes: batch, KV heads, group size, head dim,
block size, ragged lengths (down to one token), budget or sparsity, local
and minimum counts, descriptor kind, KV dtype and the rectify interval f are
drawn per case, so combinations no hand-written case names are covered too.  Same bars as the other parity
tests: selection bit-exact (inputs carry the score gap), o within 2e-2
(1e-4 for fp32 rectify), lse within 1e-4 relative, and the rectified cache
and descriptors exact."""
import numpy as np
import pytest

import block_sparse_attention_build_amd as bsa
from harness import compare_step, enforce_gap, oracle_decode, prefill, random_page_table, to_dev
from test_gpu_parity import BF16, F32, MEAN, MINMAX, make_inputs, run_select_decode
from test_gpu_parity import test_rectify_parity as rectify_case
from test_gpu_gate import test_gated_select_decode_parity as gated_case

pytestmark = pytest.mark.gpu

N_CASES = 64
N_RECTIFY = 16
N_GATED = 16


def _draw(seed):
    rng = np.random.Generator(np.random.PCG64(9000 + seed))
    dtype = BF16 if rng.random() < 0.75 else F32
    kind = MINMAX if rng.random() < 0.7 else MEAN
    d = int(rng.choice([64, 128]))
    blk = int(rng.choice([32, 64, 128, 256]))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    B = int(rng.integers(1, 5))
    lengths = [int(x) for x in rng.integers(1, 40 * blk, size=B)]
    if rng.random() < 0.5:
        budget, bp = int(rng.integers(1, 24)) * blk, 0
    else:
        budget, bp = 0, int(rng.choice([5000, 8000, 9000, 9500]))
    n_local = int(rng.integers(1, 4))
    n_min = int(rng.integers(0, 6))
    return dtype, d, blk, kind, G * Hkv, Hkv, lengths, budget, bp, n_local, n_min


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape_select_decode(seed):
    case = _draw(seed)
    dtype, d, blk, kind, Hq, Hkv, lengths, budget, bp, nl, nm = case
    print(f"seed {seed}: {case}", flush=True)
    B = len(lengths)
    max_blocks = (max(lengths) + blk - 1) // blk + 1
    L = bsa.Layout(B, Hq, Hkv, d, blk, max_blocks, dtype, kind)
    P = bsa.SelectParams(budget_tokens=budget, sparsity_bp=bp, n_local=nl, n_min=nm)
    P.n_max = bsa.block_count(P, max_blocks, blk)
    q, Ks, Vs, Wg = make_inputs(500 + seed, B, Hq, Hkv, d, lengths, dtype, kind)
    enforce_gap(L, P, q, Ks, [[T] for T in lengths], W_gate=Wg)
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 600 + seed))
    cache.k_pool.fill_(float("nan"))
    cache.v_pool.fill_(float("nan"))
    prefill(L, cache, Ks, Vs, lengths)
    if Wg is not None:
        P.gate_w = to_dev(Wg, bsa.Layout(1, 1, 1, d, blk, 1, BF16))
    idx, cnt, o, lse = run_select_decode(L, cache, to_dev(q, L), P)
    ref = oracle_decode(P, q, Ks, Vs, lengths, L, W_gate=Wg)
    compare_step(L, idx, cnt, o, lse, ref)


def _draw_rectify(seed):
    rng = np.random.Generator(np.random.PCG64(9500 + seed))
    dtype = BF16 if rng.random() < 0.8 else F32
    d = int(rng.choice([64, 128]))
    blk = int(rng.choice([32, 64, 128, 256]))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    f = int(rng.integers(1, 129))
    while G * f > 4096:
        f //= 2
    B = int(rng.integers(1, 5))
    lengths = [int(x) for x in rng.integers(f, f + 30 * blk, size=B)]
    return dtype, d, blk, f, lengths, G * Hkv, Hkv


@pytest.mark.parametrize("seed", range(N_RECTIFY))
def test_random_shape_rectify(seed):
    case = _draw_rectify(seed)
    print(f"seed {seed}: {case}", flush=True)
    rectify_case(*case)


@pytest.mark.parametrize("seed", range(N_GATED))
def test_random_shape_gated_select_decode(seed):
    """The same draws with the log-gate bias: bias beside each kept id and the
    gated decode, against the oracle."""
    case = _draw(1000 + seed)
    print(f"seed {1000 + seed}: {case}", flush=True)
    gated_case(case)
