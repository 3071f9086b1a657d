"""Pins of the oracle's elementary pieces against things other than itself:
torch's bfloat16 conversion, published Philox known-answer vectors, exact
integer arithmetic, and statistical properties of the generator."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ bf16

def _torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_random():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    np.testing.assert_array_equal(O.bf16_rne(x), _torch_bf16_bits(x))


def test_bf16_rne_ties_and_edges():
    # exact ties (lower half 0x8000) with even and odd upper halves, values just
    # around the tie, signed zeros, subnormals, the largest finite values
    uppers = np.array([0x3f80, 0x3f81, 0xbf80, 0xbf81, 0x0000, 0x0001, 0x8000, 0x7f7f, 0xff7f,
                       0x0080, 0x007f], np.uint32)
    lowers = np.array([0x0000, 0x0001, 0x7fff, 0x8000, 0x8001, 0xffff], np.uint32)
    bits = (uppers[:, None] << 16 | lowers[None, :]).ravel()
    x = bits.view(np.float32)
    x = np.concatenate([x, np.array([np.inf, -np.inf, 0.0, -0.0], np.float32)])
    np.testing.assert_array_equal(O.bf16_rne(x), _torch_bf16_bits(x))


def test_bf16_to_f32_matches_torch():
    h = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = O.bf16_to_f32(h)
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))


# ------------------------------------------------------------------ RNG

def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        ctr = [int(x, 16) for x in v["ctr"]]
        key = [int(x, 16) for x in v["key"]]
        out = [int(x, 16) for x in v["out"]]
        assert [int(x) for x in O.philox4x32_10(ctr, key)] == out


def test_pcg_hash_is_a_bijection_on_a_range():
    x = np.arange(1 << 22, dtype=np.uint32) * np.uint32(2654435761)  # spread over 2^32
    h = O.pcg_hash(x)
    assert np.unique(h).size == x.size


def test_xi16_is_uniform_and_independent_of_parity():
    # chi-square over 256 bins of the top byte, both halves, 2^20 samples
    u = np.concatenate([O.xi16(42, t, j, 0, 16384) for t in (1, 2) for j in range(32)])
    assert u.max() < 65536
    for half in (u[0::2], u[1::2]):
        counts = np.bincount(half >> 8, minlength=256)
        e = half.size / 256
        chi2 = ((counts - e) ** 2 / e).sum()
        # 255 dof: mean 255, sd ~22.6; 6 sd bound
        assert chi2 < 255 + 6 * 22.6, chi2
    # lag-1 correlation between consecutive elements is ~0
    a = u[:-1].astype(np.float64) - 32767.5
    b = u[1:].astype(np.float64) - 32767.5
    r = (a * b).mean() / a.var()
    assert abs(r) < 6 / np.sqrt(a.size)


def test_xi16_keys_on_seed_step_block_and_element():
    base = O.xi16(42, 3, 7, 0, 4096)
    for other in (O.xi16(43, 3, 7, 0, 4096), O.xi16(42, 4, 7, 0, 4096), O.xi16(42, 3, 8, 0, 4096),
                  O.xi16(42, 3, 7, 2, 4096)):
        assert (other == base).mean() < 0.01
    # element-wise definition: element i of a run from local0 equals the single call
    assert int(O.xi16(42, 3, 7, 5, 1)[0]) == int(O.lib().orc_xi16(42, 3, 7, 5))


# ------------------------------------------------------------------ blocks and quotas

CONFIG_D = {
    # flat parameter counts of the five synthetic workloads: the weight matrices of each
    # architecture (attention 4·h², MLP 2 or 3 matrices, embeddings), biases and norms left out
    "tiny": 2**20,
    "bert_base": 12 * (4 * 768 * 768 + 2 * 768 * 3072) + 30522 * 768,
    "opt_1_3b": 24 * (4 * 2048 * 2048 + 2 * 2048 * 8192) + 50272 * 2048,
    "llama2_7b": 32 * (4 * 4096 * 4096 + 3 * 4096 * 11008) + 2 * 32000 * 4096,
    "llama2_13b": 40 * (4 * 5120 * 5120 + 3 * 5120 * 13824) + 2 * 32000 * 5120,
}


@pytest.mark.parametrize("name", list(CONFIG_D))
def test_quota_is_exact_and_telescopes(name):
    d = CONFIG_D[name]
    B = 16384
    k = d // 100
    cfg = O.make_cfg(d, B, k, 10)
    nb = O.num_blocks(cfg)
    assert nb == -(-d // B)
    rng = np.random.default_rng(1)
    js = np.unique(np.concatenate([[0, nb - 1], rng.integers(0, nb, 300)]))
    for j in js:
        off, kb = O.block_quota(cfg, j)
        s, n = O.block_range(cfg, j)
        assert off == (k * s) // d          # Python integers are exact
        assert kb == (k * (s + n)) // d - (k * s) // d
        assert 0 <= kb <= n
    last_off, last_kb = O.block_quota(cfg, nb - 1)
    assert last_off + last_kb == k


def test_quota_value_counts_tiny_and_bert():
    # every block: the quotas sum to k and take the two values around B*k/d
    for d in (CONFIG_D["tiny"], CONFIG_D["bert_base"]):
        cfg = O.make_cfg(d, 16384, d // 100, 10)
        nb = O.num_blocks(cfg)
        kbs = np.array([O.block_quota(cfg, j)[1] for j in range(nb)])
        assert kbs.sum() == d // 100
        full = kbs[:-1] if d % 16384 else kbs
        assert set(np.unique(full)) <= {163, 164}
    cfg = O.make_cfg(CONFIG_D["tiny"], 16384, 10485, 10)
    kbs = np.array([O.block_quota(cfg, j)[1] for j in range(64)])
    assert (kbs == 164).sum() == 53 and (kbs == 163).sum() == 11


def test_floor_mul_div_large():
    rng = np.random.default_rng(2)
    for _ in range(2000):
        d = int(rng.integers(1, 2**62))
        k = int(rng.integers(0, d + 1))
        x = int(rng.integers(0, d + 1))
        assert O.floor_mul_div(k, x, d) == (k * x) // d


def test_step_constants_special_values():
    cfg = O.make_cfg(1000, 100, 10, 10)
    fac1, fac2, c1, c2, decay = O.step_constants(cfg, 1)
    # t = 1: the row written now (row 1) has age 0; bias correction is exactly 1
    assert fac1[1] == 1.0 and fac2[1] == 1.0
    assert c1 == 1.0 and c2 == 1.0
    assert decay == 1.0
    # age of physical row i at step t is (t - i) mod m
    fac1, _, _, _, _ = O.step_constants(cfg, 13)
    for i in range(10):
        r = (13 - i) % 10
        assert fac1[i] == np.float32(float(np.float32(0.9)) ** r)
    cfg_wd = O.make_cfg(1000, 100, 10, 10, lr=1e-3, wd=0.1)
    assert O.step_constants(cfg_wd, 5)[4] == np.float32(1 - 1e-4)
