"""GPU parity of the final radix selection's early end (32-bit keys).

The selection may stop before the last digit once the digit holding the
remaining rank holds exactly that many keys: every key of that digit is then
in the top k, whatever its low bits.  Each row below puts a cluster of fp32
values that share every bit but the lowest few (1 + i * ulp above 2.0) at the
k-th position, with G larger values above it and smaller values below, so that
the cluster fills one digit of the second pass: when G + cluster == k the
selection ends there; otherwise a third (and fourth) pass must split the
cluster.  Clusters with repeated values make the k-th value a tie.  Every case
prints its name before its GPU step.
"""
import numpy as np
import pytest
import torch

from workloads.synth import F32, Workload
from tests.gpu_util import check_varlen, run_varlen, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

K = 1024
N = 16384
BASE = np.float32(2.0).view(np.uint32)

# (cluster size, distinct values in it, larger values above it)
ROWS = [
    (16, 16, K - 16),   # the cluster completes the rank: early end
    (16, 16, K - 5),    # five of sixteen: the low bits decide
    (64, 64, K - 64),   # early end, six low bits
    (64, 64, K - 40),
    (16, 4, K - 16),    # four values four times each: early end
    (16, 4, K - 6),     # the k-th value is a tie
    (1, 1, K - 1),
    (2, 1, K - 1),      # two equal keys, one of them taken
]


def _row(rng, size, distinct, above):
    bits = BASE + (np.arange(size) % distinct).astype(np.uint32)
    cluster = bits.view(np.float32)
    big = rng.uniform(4.0, 8.0, size=above).astype(np.float32)
    rest = rng.uniform(-1.0, 1.9, size=N - size - above).astype(np.float32)
    row = np.concatenate([cluster, big, rest])
    rng.shuffle(row)
    return row


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_select_range_clusters(seed):
    rng = np.random.default_rng(9100 + seed)
    x = np.stack([_row(rng, *spec) for spec in ROWS]).view(np.uint32)
    # a gaussian control row
    x = np.concatenate([x, rng.standard_normal((1, N), dtype=np.float32).view(np.uint32)])
    R = x.shape[0]
    wl = Workload(name="select-range", kind="varlen", dtype=F32, x=x, width=N, k=K,
                  seq_lens=np.full(R, N, np.int32), next_n=1, compress_ratio=1,
                  pre_idx=None, return_values=True)
    say(f"select range clusters seed {seed}: {R} rows x {N} fp32, top_k {K}")
    idx, vals, _ = run_varlen(wl)
    errs = check_varlen(wl, idx, vals)
    assert errs == [], "\n".join(errs[:8])
