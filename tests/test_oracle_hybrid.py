"""Pins of the oracle's hybrid stack (the 74B preview's hybrid_sliding blocks, every other
block windowed): a window that covers the sequence changes nothing; window_layers 1
windows blocks 0, 2, ... and 2 windows blocks 1, 3, ... (checked through which layer first
departs from the full-attention stack, and only on tokens past the window)."""
import numpy as np

from oracle import zaya_oracle as O
from tests.test_oracle_pins import npw, tiny
from zaya_synth import block_weights, stack_weights, token_ids

W = 3


def _stack(cfg):
    sw = npw(stack_weights(cfg))
    blocks = [npw(block_weights(cfg, i)) for i in range(cfg.num_layers)]
    return O.stack_forward(cfg, sw, lambda i: blocks[i], token_ids(cfg).numpy())


def _cfg(**kw):
    return tiny(name="tiny_hybrid", seq=10, num_layers=3, **kw)


def test_window_covering_the_sequence_is_full_attention():
    full = _stack(_cfg())
    for wl in (0, 1, 2):
        cov = _stack(_cfg(sliding_window=9, window_layers=wl))
        for a, b in zip(full["layer_outputs"], cov["layer_outputs"]):
            np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(full["logits"], cov["logits"])


def test_window_layers_pick_alternate_blocks():
    full = _stack(_cfg())
    even = _stack(_cfg(sliding_window=W, window_layers=1))  # blocks 0 and 2 windowed
    odd = _stack(_cfg(sliding_window=W, window_layers=2))  # block 1 windowed
    every = _stack(_cfg(sliding_window=W, window_layers=0))
    f0, e0, o0, a0 = (r["layer_outputs"][0][0] for r in (full, even, odd, every))
    # block 0: windowed under 1 and 0, full under 2; tokens t <= W see their whole prefix anyway
    np.testing.assert_array_equal(o0, f0)
    np.testing.assert_array_equal(e0, a0)
    np.testing.assert_array_equal(e0[:W + 1], f0[:W + 1])
    assert not np.allclose(e0[W + 1:], f0[W + 1:])
    # under 2 the first departure is in block 1
    assert not np.allclose(odd["layer_outputs"][1][0][W + 1:], full["layer_outputs"][1][0][W + 1:])
    # block 1 of a window_layers-1 stack attends fully: it equals a full block on block 0's
    # windowed output and router state
    cfg = _cfg(sliding_window=W, window_layers=1)
    b1 = npw(block_weights(cfg, 1))
    ref = O.block_forward(cfg.replace(sliding_window=-1), b1, even["layer_outputs"][0], even["router_states"][0])
    np.testing.assert_array_equal(ref["layer_output"], even["layer_outputs"][1].reshape(-1, cfg.hidden_size))
