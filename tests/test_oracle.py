"""The fp64 oracle against facts that do not come from the oracle itself."""
import math

import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS, _randn


def oracle_fwd(q, k, v, scale, causal, rows=None):
    return oracle.attention_forward(q, k, v, scale, causal, rows=rows)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle_fwd)


def test_row_blocks_do_not_change_result():
    """The block of rows processed at once only bounds memory."""
    q, k, v = (_randn(300 + t, 1, 2, 300, 16) for t in range(3))
    for causal in (False, True):
        O1, L1 = oracle.attention_forward(q, k, v, 0.25, causal, row_block=7)
        O2, L2 = oracle.attention_forward(q, k, v, 0.25, causal, row_block=1000)
        assert np.max(np.abs(O1 - O2)) <= 1e-13
        assert np.max(np.abs(L1 - L2)) <= 1e-13


def test_scale_is_rounded_to_float32():
    """The library takes the scale as a float32; the oracle uses that value."""
    s = 1.0 / math.sqrt(128.0)
    assert oracle.boundary_scale(s) == float(np.float32(s))
    assert oracle.boundary_scale(s) != s


def test_empty_shapes():
    for shape in [(0, 1, 4, 8), (1, 0, 4, 8), (1, 1, 0, 8)]:
        z = np.zeros(shape)
        O, L = oracle.attention_forward(z, z, z, 1.0, True)
        assert O.shape == shape and L.shape == shape[:3]


def test_bfloat16_inputs_upcast_exactly():
    torch = pytest.importorskip("torch")
    x = torch.randn(1, 1, 9, 8).to(torch.bfloat16)
    assert np.array_equal(oracle.as_f64(x), x.double().numpy())
    O, _ = oracle.attention_forward(x, x, x, 0.5, False)
    O2, _ = oracle.attention_forward(x.double().numpy(), x.double().numpy(),
                                     x.double().numpy(), 0.5, False)
    assert np.array_equal(O, O2)


# --- online softmax (FlashAttention, Playable, EP 04) -----------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile", [1, 3, 7, 16, 10_000])
def test_streaming_equals_two_pass(tile, causal):
    """Tile-by-tile online softmax reaches the two-pass result to 1e-12."""
    q, k, v = (_randn(400 + t, 1, 2, 37, 8) for t in range(3))
    O1, L1 = oracle.attention_forward(q, k, v, 0.8, causal)
    O2, L2 = oracle.streaming_attention(q, k, v, 0.8, causal, tile=tile)
    assert np.max(np.abs(O1 - O2)) <= 1e-12
    assert np.max(np.abs(L1 - L2)) <= 1e-12


def _growing_max_inputs(N=256, d=16, seed=7):
    """Small replica of the rescale-stress recipe: K row j scaled by
    1 + 3*j/N so later tiles carry larger score maxima; V ~ U(-1, 1)."""
    rng = np.random.default_rng([seed, 0])
    q = rng.standard_normal((1, 1, N, d)) * 2.0
    k = rng.standard_normal((1, 1, N, d)) * (1 + 3 * np.arange(N) / N)[:, None]
    v = rng.uniform(-1, 1, size=(1, 1, N, d))
    return q, k, v


def test_streaming_without_rescale_is_wrong_when_max_grows():
    """Skipping the rescale silently corrupts the result once a later tile
    brings a larger maximum (EP 04's failing streamer)."""
    q, k, v = _growing_max_inputs()
    O, L = oracle.attention_forward(q, k, v, 0.25, True)
    Ob, Lb = oracle.streaming_attention(q, k, v, 0.25, True, tile=16,
                                        rescale=False)
    Og, _ = oracle.streaming_attention(q, k, v, 0.25, True, tile=16)
    assert np.max(np.abs(Og - O)) <= 1e-12
    assert np.max(np.abs(Ob - O)) > 0.1
    rel = np.linalg.norm(Ob - O, axis=-1) / np.linalg.norm(O, axis=-1)
    assert np.max(rel) > 0.4


def test_streaming_without_rescale_harmless_when_first_tile_holds_max():
    """If the first tile already holds every row's maximum, no rescale is
    ever needed and the failing streamer happens to be right."""
    N, d = 48, 4
    q, k, v = (_randn(500 + t, 1, 1, N, d) for t in range(3))
    q[..., 0] = 1.0
    q[..., 1:] = 0.0
    k[0, 0, :, 0] = np.linspace(0, -3, N)  # scores fall along the sequence
    O, L = oracle.attention_forward(q, k, v, 1.0, False)
    Ob, Lb = oracle.streaming_attention(q, k, v, 1.0, False, tile=8,
                                        rescale=False)
    assert np.max(np.abs(Ob - O)) <= 1e-12
    assert np.max(np.abs(Lb - L)) <= 1e-12
