"""Shared-prefix decode (pa_decode_shared_prefix) on the GPU against the fp64
oracle.  The result is defined exactly as pa_decode's: the shared prompt
blocks change only how often they are read, so the reference is the oracle's
plain decode over each sequence's whole context.

Tolerance: bf16 inputs |gpu - ref| <= 2e-2 + 2e-2|ref| (the only dtype the
shared-prefix path is built for).  Pools are NaN-poisoned before any write.
"""

import numpy as np
import pytest

import oracle
from workloads import make_decode, make_tiny_shared

from gpu_util import (assert_close, gpu_decode, gpu_pool_for, gpu_shared_prefix, log, oracle_pools,
                      shared_prefix_workspace, to_f64)

pytestmark = pytest.mark.gpu


def _oracle_decode(wl, seqs=None):
    pk, pv = oracle_pools(wl, oracle)
    return oracle.decode(wl.q, pk, pv, wl.block_tables, wl.context_lens, wl.scale, wl.dtype,
                         seqs=seqs)


def _check_shared_tables(wl, group_size, prefix_lens):
    """The call's precondition: a group's tables agree over its prefix."""
    for g, pl in enumerate(prefix_lens):
        rows = wl.block_tables[g * group_size:(g + 1) * group_size, : int(pl) // 16]
        assert (rows == rows[0]).all()


SHAPES = [
    # n_prompts, samples, prompt_len, tails, Hq, Hkv, D
    (2, 3, 32, (1, 5, 16, 17, 3, 30), 4, 2, 64),
    (3, 4, 160, (1, 2, 15, 16, 17, 40, 64, 65, 100, 7, 33, 1), 32, 8, 128),
    (2, 2, 48, (9, 16, 1, 200), 8, 8, 128),   # G = 1
    (2, 8, 64, tuple(range(1, 17)), 16, 2, 128),  # G = 8, 8 samples
    (1, 5, 1024, (3, 70, 130, 1, 16), 8, 4, 64),  # long prefix: several prefix partitions
]


@pytest.mark.parametrize("n_prompts,samples,prompt_len,tails,Hq,Hkv,D", SHAPES)
def test_shared_prefix_shapes(n_prompts, samples, prompt_len, tails, Hq, Hkv, D):
    log(f"shared prefix {n_prompts}x{samples} prompt {prompt_len} Hq {Hq} Hkv {Hkv} D {D}")
    wl = make_tiny_shared(seed=31 + prompt_len, n_prompts=n_prompts, samples=samples,
                          prompt_len=prompt_len, tails=tails, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16")
    prefix = [prompt_len] * n_prompts
    _check_shared_tables(wl, samples, prefix)
    pool = gpu_pool_for(wl)
    got = to_f64(gpu_shared_prefix(wl, pool, samples, prefix))
    ref = _oracle_decode(wl)
    assert_close(got, ref, "bf16", "shared prefix")
    # and the plain decode on the same inputs agrees with it
    assert_close(got, to_f64(gpu_decode(wl, pool)), "bf16", "shared prefix vs pa_decode")


@pytest.mark.parametrize("declared", ["shorter", "zero", "mixed"])
def test_declared_prefix_may_be_shorter_than_shared(declared):
    """Declaring fewer shared tokens than the tables share is valid: the rest
    is read per sequence.  A zero prefix is the plain decode."""
    log(f"shared prefix declared={declared}")
    wl = make_tiny_shared(seed=5, n_prompts=3, samples=2, prompt_len=64, tails=(3, 9, 1, 17, 20, 5),
                          Hq=8, Hkv=2, D=128, dtype="bf16")
    prefix = {"shorter": [48, 48, 48], "zero": [0, 0, 0], "mixed": [64, 16, 0]}[declared]
    got = to_f64(gpu_shared_prefix(wl, gpu_pool_for(wl), 2, prefix, max_prefix=64))
    assert_close(got, _oracle_decode(wl), "bf16", f"declared {declared}")


def test_workspace_reused_and_larger_bound():
    """A workspace from an earlier call (stale contents) and a host bound above
    every prefix give the same result as a fresh call."""
    log("shared prefix workspace reuse")
    wl = make_tiny_shared(seed=9, n_prompts=2, samples=4, prompt_len=96,
                          tails=(1, 2, 3, 4, 50, 60, 70, 80), Hq=8, Hkv=2, D=128, dtype="bf16")
    pool = gpu_pool_for(wl)
    S, Hq, D = wl.q.shape
    ws = shared_prefix_workspace(S, Hq, wl.num_kv_heads, D, int(wl.context_lens.max()), 4, 96)
    ws.fill_(float("nan"))
    a = to_f64(gpu_shared_prefix(wl, pool, 4, [96, 96], workspace=ws))
    b = to_f64(gpu_shared_prefix(wl, pool, 4, [96, 96], workspace=ws))
    assert np.array_equal(a, b)
    c = to_f64(gpu_shared_prefix(wl, pool, 4, [96, 96], max_prefix=144))
    assert_close(c, _oracle_decode(wl), "bf16", "larger bound")


def test_config4_shared_prefix_full():
    """The shared-prefix batch at full size: 32 prompts x 4 samples, 2048-token
    prompts, tails U[1, 256]; every sequence against the oracle."""
    log("shared prefix config 4 (full)")
    wl = make_decode(4)
    prefix = [wl.extra["prompt_len"]] * 32
    _check_shared_tables(wl, 4, prefix)
    out = to_f64(gpu_shared_prefix(wl, gpu_pool_for(wl), 4, prefix))
    err = assert_close(out, _oracle_decode(wl), "bf16", "config 4 shared prefix")
    log(f"  max abs err {err:.3g}")