"""Gumbel-max sampler on the GPU against the oracle (same Philox stream, same
fp32 decision), plus the distribution the kernel itself draws from.

The kernel takes log2 and the reciprocal in hardware (each within about an
ulp), the oracle exactly rounded; the two may therefore pick different indices
only where two keys of a row nearly tie. Every disagreement must be such a
tie: the exact (fp64) keys of the two indices within 4e-7 relative."""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle.sampler as osm
import paged_kv_cache_slot_amd as pa
from tests.gpu_common import DEV, require_gpu, say

pytestmark = pytest.mark.gpu
NEAR_TIE = 4e-7


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def gpu_sample(probs, seed, offset):
    B = probs.shape[0]
    tok = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    pa.pa_sample_gumbel(tok, probs, seed, offset)
    torch.cuda.synchronize()
    return tok.cpu().numpy()


def check_rows(gpu_tok, probs_cpu, rows, seed, offset, what):
    """gpu_tok: tokens of `rows`; probs_cpu: the [len(rows), V] fp32 rows."""
    want, _, key64 = osm.sample(probs_cpu, seed, offset, rows=rows)
    diff = np.flatnonzero(gpu_tok != want)
    for r in diff:
        g, o = int(gpu_tok[r]), int(want[r])
        assert 0 <= g < probs_cpu.shape[1], f"{what}: row {rows[r]} index {g} out of range"
        kg, ko = key64[r, g], key64[r, o]
        assert abs(kg - ko) <= NEAR_TIE * max(kg, ko), \
            f"{what}: row {rows[r]} gpu {g} (key {kg}) oracle {o} (key {ko}) not a near-tie"
    say(f"  {what}: {len(rows)} rows, {len(diff)} near-tie disagreements")
    return len(diff)


def softmax_rows(B, V, gen, temps):
    logits = torch.randn(B, V, generator=gen, device=DEV)
    t = torch.tensor(temps, device=DEV).repeat((B + len(temps) - 1) // len(temps))[:B, None]
    return torch.softmax(logits / t, dim=1).contiguous()


@pytest.mark.parametrize("V", [1, 3, 7, 1023, 1024, 1025, 5000, 65537])
def test_small_vocab_all_rows(V):
    gen = torch.Generator(device=DEV).manual_seed(V)
    B = 9
    say(f"[case] sampler B={B} V={V}")
    probs = softmax_rows(B, V, gen, [0.3, 1.0, 3.0])
    probs[0].zero_()                                 # all zeros -> 0
    probs[1].zero_(); probs[1, V - 1] = 1.0          # one-hot at the last index
    probs[2] *= 1e-30                                # tiny, unnormalised
    tok = gpu_sample(probs, seed=11 + V, offset=3)
    assert tok[0] == 0 and tok[1] == V - 1
    n = check_rows(tok, probs.cpu().numpy(), np.arange(B), 11 + V, 3, f"V={V}")
    assert n <= 1


def test_full_size_sampled_rows():
    """256 rows of a Qwen3-sized vocabulary (151936), checked on 24 rows."""
    B, V = 256, 151936
    gen = torch.Generator(device=DEV).manual_seed(151936)
    probs = softmax_rows(B, V, gen, [0.5, 0.8, 1.0, 1.5, 3.0])
    say(f"[case] sampler full size B={B} V={V}")
    tok = gpu_sample(probs, seed=0xDEADBEEFCAFE, offset=2**33 + 5)
    rows = np.random.default_rng(0).choice(B, size=24, replace=False)
    check_rows(tok[rows], probs[rows].cpu().numpy(), rows, 0xDEADBEEFCAFE, 2**33 + 5,
               "B=256 V=151936")


def test_row_stride_and_padding_not_read():
    B, V, S = 6, 1030, 1040
    gen = torch.Generator(device=DEV).manual_seed(5)
    full = torch.rand(B, S, generator=gen, device=DEV)
    full[:, V:] = 1e30                                # would win if read
    probs = full[:, :V]
    say(f"[case] sampler strided rows B={B} V={V} stride={S}")
    tok = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    pa.pa_sample_gumbel(tok, probs, 77, 0)
    torch.cuda.synchronize()
    t = tok.cpu().numpy()
    assert (t < V).all()
    check_rows(t, probs.cpu().numpy(), np.arange(B), 77, 0, "strided")


def test_deterministic_and_offset_dependent():
    B, V = 64, 4096
    probs = torch.full((B, V), 1.0 / V, device=DEV)
    a = gpu_sample(probs, 3, 10)
    b = gpu_sample(probs, 3, 10)
    c = gpu_sample(probs, 3, 11)
    assert np.array_equal(a, b)
    assert (a != c).mean() > 0.9


def test_kernel_draws_from_p():
    """The kernel's own draws, 65535 rows x 4 offsets: frequencies fit p."""
    p = torch.tensor([0.4, 0.3, 0.15, 0.1, 0.05, 0.0, 0.0, 0.0, 0.0], device=DEV)
    B = 65535
    probs = p.repeat(B, 1).contiguous()
    counts = np.zeros(len(p), np.int64)
    for off in range(4):
        counts += np.bincount(gpu_sample(probs, 99, off), minlength=len(p))
    n = counts.sum()
    assert counts[5:].sum() == 0
    p64 = p[:5].cpu().double().numpy()
    expected = n * p64 / p64.sum()
    chi2, pval = stats.chisquare(counts[:5], expected)
    say(f"  draws {counts[:5].tolist()} expected {np.round(expected).tolist()} p-value {pval:.3g}")
    assert pval > 1e-4
