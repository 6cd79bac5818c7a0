"""CPU tests of the Learned-schedule parameter map (no kernel launches)."""
import numpy as np
import torch

from fibonacci_offset_dilated_amd.autograd import LearnedDilation, _alpha_value


def test_theta_map_init_range_and_derivative():
    m = LearnedDilation()
    assert float(m.alpha().item()) == 1.0  # theta = 0: the pages' init alpha = 1
    for t in (-40.0, -1.0, 0.25, 3.0, 40.0):
        with torch.no_grad():
            m.theta.fill_(t)
        a = float(m.alpha().item())
        assert 0.5 <= a <= 1.5
    with torch.no_grad():
        m.theta.fill_(0.7)
    m.alpha().sum().backward()
    assert abs(float(m.theta.grad.item()) - 0.5 * (1 - np.tanh(0.7) ** 2)) < 1e-6


def test_alpha_value():
    assert _alpha_value(1.5) == np.float32(1.5)
    assert _alpha_value(torch.tensor([0.75])) == np.float32(0.75)
