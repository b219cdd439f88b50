"""santa_decode_noalloc (the library's static device scratch, no allocation) against santa_decode_ex with a
caller workspace: identical kernels, so outputs and indices must be bit-identical. Two calls in a row, the
second on a smaller input, so the second call runs on scratch the first left behind."""

import pytest
import torch

import stochastic_sparse_attention_split_amd as santa
import workloads
from tests.parity import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["strat", "sys", "iid", "prop", "flash"])
def test_noalloc_matches_decode_ex_on_two_calls(mode):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    dev = torch.device("cuda:0")
    cases = [(2, 16, 4, 128, 20000, 256, 31), (1, 8, 2, 64, 3001, 64, 32)]  # the second is smaller
    for (B, H, Hkv, d, nk, S, rs) in cases:
        log(f"noalloc {mode}: B{B} H{H}/{Hkv} d{d} nk{nk} S{S}")
        q, K, V, _ = workloads.make_inputs(B, H, Hkv, d, nk, dtype="bf16", spikes_per_head=4, rng_seed=rs)
        qd, Kd, Vd = q.to(dev), K.to(dev), V.to(dev)
        L = santa.samples_per_head(nk, S, mode)
        i_ref = torch.empty((B, H, L), dtype=torch.int32, device=dev)
        ref = santa.decode(qd, Kd, Vd, S, mode, 5, idx_out=i_ref)
        out = torch.full_like(ref, float("nan"))
        i_na = torch.full_like(i_ref, -1)
        santa.decode_noalloc(qd, Kd, Vd, S, mode, 5, out=out, idx_out=i_na)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (mode, B, nk)
        assert torch.equal(i_na, i_ref), (mode, B, nk)
