"""The seeded generator is deterministic and has the stated distributions."""

import hashlib

import numpy as np

import moe_inputs


def test_logits_bytes_are_portable():
    # numpy's PCG64 stream is fixed across platforms: the hash is a constant
    lg = moe_inputs.make_logits(64, 4, 0)
    assert lg.dtype == np.float32 and lg.shape == (64, 4)
    assert hashlib.sha256(lg.tobytes()).hexdigest() == LOGITS_TINY_SHA256


def test_generation_is_deterministic_and_shaped():
    w = moe_inputs.WORKLOADS["tiny_n64_h64_e4_k2"]
    a = moe_inputs.make_tensors(w, "cpu")
    b = moe_inputs.make_tensors(w, "cpu")
    for k in a:
        assert a[k].shape == b[k].shape
        assert a[k].equal(b[k])
    assert a["x"].shape == (64, 64) and a["w1"].shape == (4, 256, 64) and a["w2"].shape == (4, 64, 128)


def test_distributions():
    w = moe_inputs.WORKLOADS["small_qwen3moe_n1024_h512_e8_k2"]
    T = moe_inputs.make_tensors(w, "cpu")
    x = T["x"].double().numpy()
    w1 = T["w1"].double().numpy()
    lg = T["logits"].double().numpy()
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    assert abs(w1.std() - 0.02) < 2e-4
    assert abs(lg.std() - 1.0) < 0.03          # 8192 draws
    # weights of different experts are different draws
    assert not np.array_equal(w1[0], w1[1])


def test_skew_bias_profile():
    prof = moe_inputs.zipf_rank_profile(128, 3)
    assert np.isclose(prof.max(), 1.0) and np.isclose(np.sort(prof)[0], 128 ** -1.1)
    assert len(np.unique(prof)) == 128


LOGITS_TINY_SHA256 = "815dc0e8486f29377791bf2a7d14cbfe5a312b06d5742ee87cbf5cbe672bad79"


def test_ep_receive_order_is_the_source_major_layout():
    El, ep, C = 3, 4, 5
    p = moe_inputs.ep_receive_order(El, ep, C)
    assert p.dtype == np.int32 and sorted(p.tolist()) == list(range(El * ep * C))
    for e in range(El):
        for src in range(ep):
            for c in range(C):
                # slot (e, src, c) in expert-major order reads source src's chunk
                assert p[e * ep * C + src * C + c] == src * El * C + e * C + c

