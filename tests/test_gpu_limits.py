"""Parity at the size limits the library accepts: the largest block count
(N/bs = 65536, the widest 16-bit block id in the router's survivor lists)
and block counts beyond what the bucketing histograms in LDS (more than
16384 blocks per KV group, where the pair counts go straight to global
atomics), for the per-head router and each routing variant.  The whole layer
runs on the GPU; routing and outputs are checked on sampled rows against the
oracle, as for the full-size workloads."""
import pytest

import tests.test_gpu_consensus as C
import tests.test_gpu_cumulant as U
import tests.test_gpu_parity as P
import tests.test_gpu_tree as T
from content_routed_block_amd.workloads import Workload

pytestmark = pytest.mark.gpu

lsa = P.lsa  # the module fixture: skips without a GPU

LIMITS = [
    # 65536 blocks of 16 keys: the maximum block count, GQA-free
    Workload("limit_nb65536_bs16", 1, 1, 1, 16 * 65536, 64, 16, 16, 16, 1, "topics", topics=64,
             seed=91),
    # 20000 blocks of 32 keys over a 2:1 group, odd window-block count
    Workload("limit_nb20000_bs32", 1, 2, 1, 32 * 20000, 64, 32, 8, 96, 1, "normal", seed=92),
    # the maximum block count with 32-entry selection lists
    Workload("limit_nb65536_bs16_k32", 1, 1, 1, 16 * 65536, 64, 16, 32, 16, 1, "topics", topics=64,
             seed=93),
]


@pytest.mark.parametrize("w", LIMITS, ids=lambda w: w.name)
def test_limits_sampled_rows(lsa, w):
    P.check_sampled_rows(lsa, w, nrows=2000)


@pytest.mark.parametrize("w", LIMITS[:1], ids=lambda w: w.name)
def test_limits_consensus_sampled_rows(lsa, w):
    C.check_consensus_sampled_rows(lsa, w.replace(q_heads=2))


@pytest.mark.parametrize("w", LIMITS[:1], ids=lambda w: w.name)
def test_limits_cumulant_sampled_rows(lsa, w):
    U.check_cumulant_sampled_rows(lsa, w)


@pytest.mark.parametrize("w", LIMITS, ids=lambda w: w.name)
def test_limits_tree_sampled_rows(lsa, w):
    T.check_tree_sampled_rows(lsa, w, 8)
