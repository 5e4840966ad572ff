"""Host-side checks of the seeded input generators (no GPU)."""
import math

import numpy as np
import torch

from dynamic_sparse_attention_proxy_amd import synth
from oracle import crisp_oracle as O


def test_routing_family_is_seeded_and_graded():
    """The graded-structure family is reproducible, and under the oracle its
    first KV group (sink coupling 0, 2.5, 5, 7.5 on queries, no locality)
    orders C_struct by the sink coupling, while the heads with the strongest
    locality put more mass on the recency window than the structureless
    head does."""
    n = 2048
    a = synth.make_routing_family(seq_len=n, num_q_heads=32, num_kv_heads=8)
    b = synth.make_routing_family(seq_len=n, num_q_heads=32, num_kv_heads=8)
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    scale = 1.0 / math.sqrt(128)

    def proxy(h):
        q = a.q[h].double().numpy()
        k = a.k[h // 4].double().numpy()
        return O.proxy_map(q[n - 128:], k, scale)[0]

    c = [O.c_struct(proxy(h)) for h in range(4)]
    assert all(c[i] < c[i + 1] for i in range(3)), c
    rec0 = proxy(0)[:, -128:].sum() / 128
    rec24 = proxy(24)[:, -128:].sum() / 128
    assert rec24 > 5 * rec0, (rec0, rec24)
    assert np.isfinite(a.q.float().numpy()).all()
