"""Decode-step graphs on the GPU: every replay is checked bit for bit against
the same step run eagerly (pa_store_kvcache + pa_decode at the bucket's batch
on the same inputs), pools included, and some replays against the oracle too.
Replays alternate with eager work and synchronisations, each bucket is
replayed several times with new data, and batches that are not a bucket are
padded (context length 0, slot -1) to the next one."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_slot_amd as pa
from tests.gpu_common import DEV, compare, require_gpu, say

pytestmark = pytest.mark.gpu

HQ, HKV, D = 16, 8, 128
SCALE = 1.0 / math.sqrt(D)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


class Static:
    """Static step buffers for buckets up to B, a pool of NB blocks of bs."""

    def __init__(self, B, NB, bs, max_len, seed):
        self.B, self.NB, self.bs, self.max_len = B, NB, bs, max_len
        self.stride = -(-max_len // bs)
        g = torch.Generator(device=DEV).manual_seed(seed)
        rnd = lambda *s: torch.randn(*s, generator=g, device=DEV).to(torch.bfloat16)
        self.kc, self.vc = rnd(NB, bs, HKV, D), rnd(NB, bs, HKV, D)
        self.q, self.k_new, self.v_new = rnd(B, HQ, D), rnd(B, HKV, D), rnd(B, HKV, D)
        self.out = torch.zeros(B, HQ, D, dtype=torch.bfloat16, device=DEV)
        self.slots = torch.full((B,), -1, dtype=torch.int32, device=DEV)
        self.lens = torch.zeros(B, dtype=torch.int32, device=DEV)
        self.table = torch.full((B, self.stride), -1, dtype=torch.int32, device=DEV)
        nbytes = pa.pa_decode_workspace_bytes(B, HQ, D, max_len, bs)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        self.g = torch.Generator(device=DEV).manual_seed(seed + 1)

    def graphs(self, buckets):
        return pa.pa_decode_graphs_create(self.out, self.q, self.k_new, self.v_new, self.kc,
                                          self.vc, self.slots, self.lens, self.table, self.ws,
                                          self.max_len, SCALE, buckets=buckets)

    def fill(self, batch, bucket, rng):
        """New inputs for rows [0, bucket): `batch` live rows with distinct
        blocks per row and the new token's slot at its last position, then
        padding rows."""
        lens = rng.integers(1, self.max_len + 1, size=batch)
        lens[rng.integers(0, batch)] = self.max_len          # one row at the bound
        perm = rng.permutation(self.NB)
        table = np.full((bucket, self.stride), -1, np.int32)
        slots = np.full(bucket, -1, np.int32)
        used = 0
        for b, L in enumerate(lens):
            n = -(-int(L) // self.bs)
            table[b, :n] = perm[used:used + n]
            used += n
            slots[b] = table[b, (L - 1) // self.bs] * self.bs + (L - 1) % self.bs
        assert used <= self.NB
        full_lens = np.zeros(bucket, np.int32)
        full_lens[:batch] = lens
        self.lens[:bucket].copy_(torch.from_numpy(full_lens))
        self.slots[:bucket].copy_(torch.from_numpy(slots))
        self.table[:bucket].copy_(torch.from_numpy(table))
        for t in (self.q, self.k_new, self.v_new):
            t[:bucket].copy_(torch.randn(t[:bucket].shape, generator=self.g,
                                         device=DEV).to(torch.bfloat16))
        pa.pa_validate_metadata(table, full_lens, self.NB, self.bs, slot_mapping=slots,
                                max_context_len=self.max_len)

    def eager(self, bucket, kc, vc):
        """The same step without graphs, on copies of the pools."""
        out = torch.full((bucket, HQ, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        pa.pa_store_kvcache(self.k_new[:bucket], self.v_new[:bucket], kc, vc, self.slots[:bucket])
        pa.pa_decode(out, self.q[:bucket], kc, vc, self.table[:bucket], self.lens[:bucket],
                     self.max_len, SCALE, self.ws)
        return out


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy()


@pytest.mark.parametrize("bs,max_len", [(16, 1000), (256, 2048)])
def test_graph_replays_match_eager_bitwise(bs, max_len):
    buckets = [1, 2, 4, 8, 16, 32, 64]
    st = Static(B=64, NB=64 * (-(-max_len // bs)) + 8, bs=bs, max_len=max_len, seed=bs)
    graphs = st.graphs(buckets)
    assert graphs.buckets == tuple(buckets)
    rng = np.random.default_rng(bs)
    checked_oracle = 0
    for trial, batch in enumerate([1, 3, 8, 13, 64, 33, 2, 17, 64, 5]):
        bucket = graphs.bucket(batch)
        assert bucket == min(b for b in buckets if b >= batch)
        st.fill(batch, bucket, rng)
        kc0, vc0 = st.kc.clone(), st.vc.clone()
        say(f"[case] graph replay bs={bs} batch={batch} bucket={bucket} trial={trial}")
        graphs.launch(batch)
        torch.cuda.synchronize()
        got, kc1, vc1 = st.out[:bucket].clone(), st.kc.clone(), st.vc.clone()
        # eager work between replays: the same step on copies of the old pools
        want = st.eager(bucket, kc0, vc0)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(got), _bits(want)), "graph output differs from eager"
        assert np.array_equal(_bits(kc1), _bits(kc0)) and np.array_equal(_bits(vc1), _bits(vc0))
        assert int(got[batch:].float().abs().sum()) == 0, "padding rows must be zero"
        if trial % 3 == 0:
            ref = oracle.decode(st.q[:bucket].cpu(), kc1.cpu(), vc1.cpu(),
                                st.table[:bucket].cpu(), st.lens[:bucket].cpu(), SCALE,
                                nthreads=8)
            compare(got, ref, f"graph bs={bs} batch={batch}")
            checked_oracle += 1
    assert checked_oracle >= 3
    graphs.close()


def test_graph_same_bucket_many_replays():
    """One bucket replayed back to back with new data each time (no eager work
    in between), then every output checked against the eager step."""
    st = Static(B=32, NB=32 * 64 + 8, bs=16, max_len=1024, seed=77)
    graphs = st.graphs([32])
    rng = np.random.default_rng(77)
    outs, states = [], []
    for i in range(6):
        st.fill(32, 32, rng)
        snap = dict(q=st.q.clone(), k=st.k_new.clone(), v=st.v_new.clone(),
                    slots=st.slots.clone(), lens=st.lens.clone(), table=st.table.clone(),
                    kc=st.kc.clone(), vc=st.vc.clone())
        say(f"[case] graph back-to-back replay {i}")
        graphs.launch(32)
        outs.append(st.out.clone())
        states.append(snap)
    torch.cuda.synchronize()
    for i, (got, s) in enumerate(zip(outs, states)):
        st.q.copy_(s["q"]); st.k_new.copy_(s["k"]); st.v_new.copy_(s["v"])
        st.slots.copy_(s["slots"]); st.lens.copy_(s["lens"]); st.table.copy_(s["table"])
        kc, vc = s["kc"].clone(), s["vc"].clone()
        want = st.eager(32, kc, vc)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(got), _bits(want)), f"replay {i} differs from eager"
    graphs.close()


def test_graph_launch_bounds():
    st = Static(B=8, NB=40, bs=16, max_len=64, seed=3)
    graphs = st.graphs([2, 8])
    assert graphs.bucket(1) == 2 and graphs.bucket(3) == 8 and graphs.bucket(8) == 8
    with pytest.raises(pa.PAError):
        graphs.bucket(9)
    with pytest.raises(pa.PAError):
        graphs.launch(9)
    graphs.launch(0)                      # nothing to do
    torch.cuda.synchronize()
    graphs.close()
