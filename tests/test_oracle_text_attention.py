"""Oracle of text-augmented window attention against its pins (CPU only)."""
import numpy as np

from oracle import attention as oatt
from oracle import text_attention as otxt
from tests import oracle_pins as pins


def test_closed_form_uniform_attention():
    pins.check_text_closed_form(otxt.text_window_attention)


def test_brute_force_sdpa_twin():
    pins.check_text_brute_force(otxt.text_window_attention)


def test_isolation():
    pins.check_text_isolation(otxt.text_window_attention)


def test_no_text_is_window_attention():
    rng = np.random.default_rng(9)
    cu = [0, 5, 5, 12]
    q, k, v = (rng.standard_normal((2, 12, 3, 8)) for _ in range(3))
    empty = np.zeros((2, 0, 3, 8))
    o, text, _ = otxt.text_window_attention(q, k, v, cu, empty, empty, empty)
    ref, _ = oatt.window_attention(q, k, v, cu)
    assert np.allclose(o, ref, rtol=0, atol=1e-14) and text.shape == (2, 0, 3, 8)
