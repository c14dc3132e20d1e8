"""Host-side checks of the seeded input generators (no method arithmetic there)."""
import numpy as np

import kda_synth as ks


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, -2.5, 65504.0, 1e-40], dtype=np.float32)
    y = ks.bf16_round(x)
    assert y[0] == 1.0
    assert y[1] == 1.0                      # tie -> even mantissa
    assert y[2] == np.float32(1 + 2**-6)    # tie -> even (rounds up)
    assert y[3] == -2.5
    assert (y.view(np.uint32) & 0xFFFF).max() == 0


def test_generators_are_seeded_and_shaped():
    a = ks.make("layer", T=128, H=2)
    b = ks.make("layer", T=128, H=2)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.g, b.g)
    assert a.q.shape == (1, 128, 2, 128) and a.beta.shape == (1, 128, 2)
    assert (a.q.view(np.uint32) & 0xFFFF).max() == 0     # bf16-exact
    v = ks.make("varlen", n_seqs=5, min_len=3, max_len=70, H=2)
    assert v.cu_seqlens[0] == 0 and v.cu_seqlens[-1] == v.T
    assert (v.state_indices == -1).sum() == 2
    valid = v.state_indices[v.state_indices >= 0]
    assert len(set(valid.tolist())) == len(valid)
    g = ks.make("gqa", B=2, T=64, Hk=2, Hv=8)
    assert g.q.shape == (2, 64, 2, 128) and g.v.shape == (2, 64, 8, 128) and g.safe_gate
    s = ks.make("segment", T=64, H=2)
    pp = ks.preceding_summary_inputs(s)
    assert pp.T == 7 * 16 and pp.cu_seqlens[-1] == pp.T
