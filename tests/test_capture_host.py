"""Host-side argument checks of the statistics capture (no GPU needed)."""
import pytest
import torch

import post_weight_quantization_amd as kq


def test_capture_rejects_cpu_layers_and_bad_counts():
    layer = torch.nn.Linear(16, 8)
    with pytest.raises(ValueError, match="GPU"):
        kq.CovarianceCapture(layer, 64)
    with pytest.raises(ValueError, match="n_total"):
        kq.CovarianceCapture(layer, 0)
