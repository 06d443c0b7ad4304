"""The seeded input generator: determinism, per-expert regeneration, distributions."""
import torch

from mixture_experts_layer_14_amd import inputs

SMALL = inputs.MoeShape("s", tokens=33, dim=256, n_experts=16, n_groups=4, topk_groups=2, topk=4,
                        inter=128, n_shared=1, route_scale=2.5, dtype="bf16", hot_bias=0.5)


def test_deterministic_and_seed_sensitive():
    a = inputs.generate(SMALL, seed=0)
    b = inputs.generate(SMALL, seed=0)
    c = inputs.generate(SMALL, seed=1)
    for n in ["x", "w_gate", "bias", "w1", "w3", "w2", "ws1", "ws3", "ws2"]:
        assert torch.equal(getattr(a, n), getattr(b, n))
        assert not torch.equal(getattr(a, n), getattr(c, n))
    assert torch.equal(inputs.regenerate_x(SMALL, seed=0), a.x)


def test_expert_regeneration_matches_bulk():
    a = inputs.generate(SMALL, seed=3)
    w1, w3, w2, *_ = inputs.expert_weights(SMALL, 7, seed=3)
    assert torch.equal(w1, a.w1[7]) and torch.equal(w3, a.w3[7]) and torch.equal(w2, a.w2[7])
    f8 = SMALL.replace(dtype="fp8")
    b = inputs.generate(f8, seed=3)
    w1, w3, w2, s1, s3, s2 = inputs.expert_weights(f8, 5, seed=3)
    assert torch.equal(w1.view(torch.uint8), b.w1[5].view(torch.uint8)) and torch.equal(s2, b.s2[5])


def test_distributions_and_hot_bias():
    big = SMALL.replace(dim=1024, inter=512, tokens=256)
    t = inputs.generate(big, seed=0)
    assert t.x.dtype == torch.bfloat16 and t.w1.dtype == torch.bfloat16 and t.bias.dtype == torch.float32
    assert abs(t.x.float().std().item() - 1.0) < 0.02
    assert abs(t.w1.float().std().item() * 1024 ** 0.5 - 1.0) < 0.02
    assert abs(t.w2.float().std().item() * 512 ** 0.5 - 1.0) < 0.02
    plain = t.bias.clone()
    plain[0::8] -= 0.5
    assert plain.min() >= -0.1 and plain.max() <= 0.1
    assert (t.bias[0::8] > 0.39).all()


def test_fp8_weights_blocks():
    f8 = SMALL.replace(dtype="fp8")
    t = inputs.generate(f8, seed=0)
    assert t.w1.dtype == torch.float8_e4m3fn and t.s1.shape == (16, 1, 2) and t.s2.shape == (16, 2, 1)
    assert t.x.dtype == torch.bfloat16 and t.w_gate.dtype == torch.bfloat16
    # every 128x128 block uses the full e4m3 range: its largest code is 448
    blk = t.w1.float().abs().view(16, 1, 128, 2, 128).amax(dim=(2, 4))
    assert torch.equal(blk, torch.full_like(blk, 448.0))
