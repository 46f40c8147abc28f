"""The seeded input generators: determinism and the value sets each workload prescribes."""
import numpy as np
import torch

import synth


def test_integer_workload_values():
    li = synth.workload_layer(0, 0, L=256)
    q = li.q_idx.float().numpy()
    assert q.shape == (256, 8, 64) and np.all(q == np.round(q)) and q.min() >= -4 and q.max() <= 4
    assert set(np.unique(li.w.float().numpy()).tolist()) <= {-1.0, -0.5, 0.5, 1.0}
    assert li.q.shape == (256, 16, 576) and li.latent.shape == (256, 576)


def test_generation_is_deterministic():
    a = synth.workload_layer(1, 3, L=64)
    b = synth.workload_layer(1, 3, L=64)
    c = synth.workload_layer(1, 4, L=64)
    assert torch.equal(a.q_idx, b.q_idx) and torch.equal(a.latent, b.latent)
    assert not torch.equal(a.q_idx, c.q_idx)


def test_fp8_rows_quantisation():
    li = synth.make_layer(32, 32, 4, 16, 2, wid=4, layer=0, qk_dtype="fp8")
    assert li.q_idx.dtype == torch.float8_e4m3fn and li.q_scale.shape == (32, 4)
    deq = li.q_idx.float() * li.q_scale[..., None]
    # every row reaches +-448 at its max-magnitude element
    assert torch.all(li.q_idx.float().abs().amax(-1) == 448.0)
    assert torch.all(deq.abs().amax(-1) > 0)


def test_decode_lengths_in_range():
    lens = synth.decode_lengths()
    assert lens.shape == (8,) and lens.min() >= 150000 and lens.max() <= 200000
    assert np.array_equal(lens, synth.decode_lengths())
