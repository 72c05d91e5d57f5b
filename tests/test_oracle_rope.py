"""Oracle window-local 3D RoPE against its pins (CPU only)."""
import numpy as np
import pytest

from oracle import plan as oplan
from oracle import rope as orope
from tests import oracle_pins as pins


def test_worked_rotations():
    pins.check_rope_worked_example(orope.rotate)


def test_worked_positions():
    pins.check_rope_positions(orope.window_local_positions, oplan)


@pytest.mark.parametrize("rope_dim,head_dim", [(12, 14), (128, 128), (60, 64), (126, 128)])
def test_rotation_properties(rope_dim, head_dim):
    pins.check_rope_properties(orope.rotate, rope_dim, head_dim)


def test_windows_restart_at_zero():
    pins.check_rope_window_restart(orope.window_local_positions, oplan)


def test_rows_rotate_every_head_alike_and_values_pass_through_span():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 3, 4, 128))
    pos = [(0, 0, 0), (7, 2, 5), (1, 14, 26)]
    y = orope.rope_rows(x, pos, 128)
    assert np.array_equal(y[:, 0], x[:, 0])          # position 0 is the identity
    for j in range(3):
        for b in range(2):
            for h in range(4):
                assert np.allclose(y[b, j, h], orope.rotate(x[b, j, h], pos[j], 128), rtol=0, atol=1e-15)
    assert np.array_equal(y[..., 126:], x[..., 126:])
