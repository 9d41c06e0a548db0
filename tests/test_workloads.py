"""The seeded input generator: determinism, bf16 rounding, shapes, skew."""
import numpy as np
import torch

from workloads import WORKLOADS, bf16_bits_to_f32, custom, f32_to_bf16_bits, make


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8,
                                  65504.0, 1e-30, -0.0, 0.0], dtype=np.float32)])
    ours = f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_deterministic_and_expert_independent():
    a = make("tiny_fp32")
    b = make("tiny_fp32")
    assert np.array_equal(a.x, b.x) and np.array_equal(a.logits, b.logits)
    for e in (0, 7):
        for u, v in zip(a.expert_weights(e), b.expert_weights(e)):
            assert np.array_equal(u, v)
    c = make("tiny_fp32", seed=1)
    assert not np.array_equal(a.x, c.x)


def test_decode_and_prefill_share_expert_weights():
    a = custom(T=4, d=32, f=16, E=4, k=2, dtype="bf16", seed=3)
    b = custom(T=40, d=32, f=16, E=4, k=2, dtype="bf16", seed=3, logit_bias="zipf")
    for u, v in zip(a.expert_weights(2), b.expert_weights(2)):
        assert np.array_equal(u, v)


def test_shapes_and_scales():
    wl = custom(T=16, d=256, f=512, E=4, k=2, dtype="f32", seed=0)
    w1, w3, w2 = wl.expert_weights(1)
    assert w1.shape == (256, 512) and w3.shape == (256, 512) and w2.shape == (512, 256)
    assert abs(w1.std() - 1 / 16) < 0.002 and abs(w2.std() - 1 / np.sqrt(512)) < 0.002


def test_zipf_skew_spans_about_100x():
    wl = make("dsv3_prefill_zipf")
    top1 = wl.logits.argmax(axis=1)
    assert top1.min() == 0   # the bias favours low expert ids
    assert wl.logits.shape == (8192, 256)


def test_named_workloads_exist():
    assert set(WORKLOADS) == {"tiny_fp32", "mixtral_prefill", "dsv3_decode", "dsv3_prefill_zipf",
                              "ep_rank_share"}


def test_regenerating_an_expert_twice_gives_same_bits():
    wl = custom(T=4, d=16, f=8, E=3, k=1, dtype="bf16", seed=2)
    for u, v in zip(wl.expert_weights(1), wl.expert_weights(1)):
        assert np.array_equal(u, v)
