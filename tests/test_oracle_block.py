"""Pins of the block-pipeline oracle: the stacked (q|k|v, gate|up) linears
reduce to the separately pinned single-linear oracle, and the adapter-only
AdamW step equals torch.optim.AdamW (CPU, float64) over several steps."""
import numpy as np
import torch

import oracle as O

B = O.block


def _lin(M, K, N, r, seed):
    rng = np.random.default_rng(seed)
    W = O.bf16_bits(rng.standard_normal((N, K)) * 0.02)
    L1 = O.bf16_bits(rng.standard_normal((K, r)) / K)
    L2 = O.bf16_bits(rng.standard_normal((r, N)) * 0.3)
    return W, L1, L2


def test_group_of_one_is_the_layer():
    rng = np.random.default_rng(1)
    M, K, N, r = 16, 128, 64, 8
    X = O.bf16_bits(rng.standard_normal((M, K)))
    dY = O.bf16_bits(rng.standard_normal((M, N)))
    W, L1, L2 = _lin(M, K, N, r, 2)
    Y, Ts = B.qlora_group_forward(X, [W], [L1], [L2], 1.5)
    Y0, T0 = O.qlora_forward(X, W, L1, L2, 1.5)
    assert np.array_equal(Y, Y0) and np.array_equal(Ts[0], T0)
    dX, dL1, dL2, G = B.qlora_group_backward(X, dY, [W], [L1], [L2], 1.5)
    r0 = O.qlora_backward(X, dY, W, L1, L2, 1.5)
    assert np.array_equal(dX, r0[0]) and np.array_equal(dL1[0], r0[1]) and np.array_equal(dL2[0], r0[2])


def test_stacked_segments_are_the_separate_layers():
    """Forward: concatenation; adapter gradients: the separate layers'; dX: the
    once-rounded sum of the separate layers' unrounded input gradients."""
    rng = np.random.default_rng(3)
    M, K, N, r, s = 24, 192, 64, 8, 2.0
    X = O.bf16_bits(rng.standard_normal((M, K)))
    lins = [_lin(M, K, N, r, 10 + g) for g in range(3)]
    dY = O.bf16_bits(rng.standard_normal((M, 3 * N)))
    Y, Ts = B.qlora_group_forward(X, *zip(*lins), s)
    for g, (W, L1, L2) in enumerate(lins):
        Yg, Tg = O.qlora_forward(X, W, L1, L2, s)
        assert np.array_equal(Y[:, g * N:(g + 1) * N], Yg) and np.array_equal(Ts[g], Tg)
    dX, dL1, dL2, G = B.qlora_group_backward(X, dY, *zip(*lins), s)
    total, slack = 0.0, 0.0
    ulp = lambda x: 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))) - 7)
    for g, (W, L1, L2) in enumerate(lins):
        dXg, dL1g, dL2g, Gg, _ = O.qlora_backward(X, dY[:, g * N:(g + 1) * N], W, L1, L2, s)
        assert np.array_equal(dL1[g], dL1g) and np.array_equal(dL2[g], dL2g) and np.array_equal(G[g], Gg)
        v = O.bf16_value(dXg)
        total = total + v                       # the separate layers' rounded input gradients, summed
        slack = slack + 0.5 * ulp(v)            # each carries at most half an ulp of rounding
    got = O.bf16_value(dX)
    assert np.all(np.abs(got - total) <= 0.5 * ulp(got) + slack)
    assert not np.allclose(got, O.bf16_value(O.qlora_backward(X, dY[:, :N], *lins[0], s)[0]), rtol=0.1)


def test_adamw_matches_torch_float64():
    rng = np.random.default_rng(5)
    n = 1000
    theta = rng.standard_normal(n) * 0.02
    m = np.zeros(n)
    v = np.zeros(n)
    p = torch.tensor(theta.copy(), dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([p], lr=2e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    for step in range(1, 6):
        g = rng.standard_normal(n) * (0.1 / step)
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        theta, m, v = B.adamw_step(theta, m, v, g, 2e-4, 0.9, 0.999, 1e-8, 0.01, step)
        st = opt.state[p]
        assert np.allclose(theta, p.detach().numpy(), rtol=1e-13, atol=1e-16)
        assert np.allclose(m, st["exp_avg"].numpy(), rtol=1e-13, atol=1e-18)
        assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=1e-20)


def test_adamw_first_step_moves_every_weight_by_lr():
    """At step 1 with no decay, m_hat = g and v_hat = g^2, so each weight moves by
    lr * g / (|g| + eps): -lr sign(g) up to eps."""
    g = np.array([1e-3, -2.0, 5.0, -1e-4])
    theta, m, v = B.adamw_step(np.zeros(4), np.zeros(4), np.zeros(4), g, 1e-3, 0.9, 0.999, 1e-12, 0.0, 1)
    assert np.allclose(theta, -1e-3 * np.sign(g), rtol=1e-7)
