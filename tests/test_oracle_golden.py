"""The stored oracle values of tests/golden/sampled_parity.npz (written by
tests/golden/make_sampled_parity.py from the oracle alone) still agree with
the oracle: the key whose gradients are cheapest to recompute in each workload
(the last live slot, a generation-copy token seen only by itself) is computed
again here, for one kv head, and the inputs' fingerprint is checked."""
import os

import numpy as np
import pytest

from block_sparse_masked_opr_amd import inputs as I
from oracle import opr_oracle as O
from tests.golden import make_sampled_parity as G

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "sampled_parity.npz")


@pytest.mark.parametrize("wl", G.workloads(), ids=lambda w: w[0])
def test_golden_matches_oracle(wl):
    name, rows, L, Hq, Hkv, D, seed = wl
    gold = dict(np.load(GOLDEN, allow_pickle=False))
    lay = O.layout(rows, L)
    slot = O.attention_order(lay, 0)
    tok_of_slot = np.argsort(slot)
    np.testing.assert_array_equal(tok_of_slot[gold[f"{name}_slots"]], gold[f"{name}_cols"])
    t = I.make_tensors(1, L, Hq, Hkv, D, seed=seed)
    np.testing.assert_allclose(G.fingerprint(t), gold[f"{name}_fingerprint"], rtol=1e-12)
    i = int(np.argmax(gold[f"{name}_slots"]))            # the last live slot
    col = gold[f"{name}_cols"][i:i + 1]
    g = Hq // Hkv
    f = {n: I.bf16_bits_to_f32(t[n]).astype(np.float64) for n in t}
    dk, dv = O.attn_cols(f["q"][:, :, :g], f["k"][:, :, :1], f["v"][:, :, :1], f["do"][:, :, :g], lay, 0, col,
                         G.THETA)
    np.testing.assert_allclose(dk[0, 0], gold[f"{name}_dk"][i, 0], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(dv[0, 0], gold[f"{name}_dv"][i, 0], rtol=1e-5, atol=1e-6)
