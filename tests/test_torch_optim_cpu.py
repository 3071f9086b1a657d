"""Argument checks of the torch.optim front end that need no GPU."""
import pytest
import torch

from memory_compressed_adaptive_amd.torch_optim import MicroAdamW


def test_rejects_cpu_parameters():
    with pytest.raises(ValueError):
        MicroAdamW([torch.nn.Parameter(torch.zeros(10))])
