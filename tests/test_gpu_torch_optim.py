"""The torch.optim front end (MicroAdamW) over parameter groups: the flat step
it runs equals the CPU oracle's on the concatenated parameters, its state
round-trips through state_dict, and it reduces a synthetic loss."""
import numpy as np
import pytest
import torch

import oracle as O
from memory_compressed_adaptive_amd.torch_optim import MicroAdamW

from gpu_harness import assert_bits_equal, assert_close_f32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SHAPES = [(64, 33), (33,), (128, 257), (7, 5, 3), (1,)]


def _params(seed, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    return [torch.nn.Parameter((torch.randn(s, generator=g) * 0.02).to(dtype).cuda()) for s in SHAPES]


def _set_grads(ps, rng):
    for p in ps:
        p.grad = torch.from_numpy((rng.standard_normal(p.numel()) * 1e-3).astype(np.float32)).reshape(p.shape).to(
            p.dtype).cuda()


def test_flat_step_matches_oracle():
    ps = _params(1)
    d = sum(p.numel() for p in ps)
    opt = MicroAdamW(ps, lr=1e-3, density=0.01, m=4, block=4096)
    theta = np.concatenate([p.detach().cpu().numpy().ravel() for p in ps]).astype(np.float32)
    orc = O.FullState(O.make_cfg(d, 4096, int(d * 0.01), 4, lr=1e-3))
    rng = np.random.default_rng(2)
    for t in range(1, 7):
        _set_grads(ps, rng)
        g32 = np.concatenate([p.grad.cpu().numpy().ravel() for p in ps]).astype(np.float32)
        say(f"[torch optim] step {t}: d={d}")
        opt.step()
        orc.step(theta, O.bf16_rne(g32))
        got = np.concatenate([p.detach().cpu().numpy().ravel() for p in ps])
        assert_close_f32(f"torch optim t={t}", got, theta)
    # the parameters are views of the group's flat buffer
    flat = opt.param_groups[0]["_flat"]
    assert ps[0].data_ptr() == flat.data_ptr()


def test_bf16_group_and_missing_grads():
    ps = _params(3, torch.bfloat16)
    d = sum(p.numel() for p in ps)
    opt = MicroAdamW(ps, lr=1e-2, weight_decay=0.1, density=0.05, m=3, block=2048)
    th16 = np.concatenate([p.detach().view(torch.int16).cpu().numpy().ravel() for p in ps]).view(np.uint16)
    orc = O.FullState(O.make_cfg(d, 2048, int(d * 0.05), 3, lr=1e-2, wd=0.1))
    rng = np.random.default_rng(4)
    for t in range(1, 5):
        _set_grads(ps, rng)
        ps[1].grad = None   # no gradient: zeros
        g = np.concatenate([(p.grad.view(torch.int16).cpu().numpy().ravel().view(np.uint16) if p.grad is not None
                             else np.zeros(p.numel(), np.uint16)) for p in ps])
        opt.step()
        orc.step_bf16(th16, g)
        got = np.concatenate([p.detach().view(torch.int16).cpu().numpy().ravel() for p in ps]).view(np.uint16)
        assert_bits_equal(f"bf16 group t={t}", got, th16)


def test_state_dict_resume():
    rng_seq = [np.random.default_rng(10 + t) for t in range(8)]
    grads = []
    for r in rng_seq:
        grads.append([(r.standard_normal(int(np.prod(s))) * 1e-3).astype(np.float32).reshape(s) for s in SHAPES])

    def run(split):
        ps = _params(5)
        opt = MicroAdamW(ps, lr=1e-3, m=3, block=4096, density=0.02)
        for t in range(8):
            if t == split:
                sd = opt.state_dict()
                ps2 = _params(5)
                for a, b in zip(ps2, ps):
                    a.data.copy_(b.data)
                opt = MicroAdamW(ps2, lr=1e-3, m=3, block=4096, density=0.02)
                opt.load_state_dict(sd)
                ps = ps2
            for p, g in zip(ps, grads[t]):
                p.grad = torch.from_numpy(g).cuda()
            opt.step()
        torch.cuda.synchronize()
        return np.concatenate([p.detach().cpu().numpy().ravel() for p in ps])

    assert_bits_equal("resume via state_dict", run(3), run(-1))


def test_reduces_a_synthetic_regression_loss():
    torch.manual_seed(0)
    X = torch.randn(512, 64, device="cuda")
    w_true = torch.randn(64, 1, device="cuda")
    y = X @ w_true
    model = torch.nn.Sequential(torch.nn.Linear(64, 64), torch.nn.Tanh(), torch.nn.Linear(64, 1)).cuda()
    opt = MicroAdamW(model.parameters(), lr=3e-3, density=0.05, m=10, block=1024)
    losses = []
    for _ in range(300):
        opt.zero_grad()
        loss = torch.nn.functional.mse_loss(model(X), y)
        loss.backward()
        opt.step()
        losses.append(float(loss.detach()))
    say(f"[torch optim] loss {losses[0]:.4f} -> {losses[-1]:.4f}")
    assert losses[-1] < 0.5 * losses[0]
