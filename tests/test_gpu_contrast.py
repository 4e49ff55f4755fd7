"""The float32 contrast beside the exact path (det-attn page, opening
measurements: a float32 online-softmax combine gives different bits for
different shard rotations; det-cross-entropy page: a float32 logsumexp over
vocabulary splits flips some token losses).  The exact path must give one
digest for every rotation and no flipped loss for any split count."""
import sys

import pytest
import torch

from bitwise_deterministic_exact_pass1_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def test_shard_rotations_float32_vs_exact():
    from bitwise_deterministic_exact_pass1_amd import attention, contrast
    say("contrast: causal GQA B=2 Hq=8 Hkv=2 S=1024 D=128 bf16, 4 shards of 256, 4 rotations")
    w = W.attn_workload("gqa_causal_bf16")
    Q, K, V = w["q"].cuda(), w["k"].cuda(), w["v"].cuda()
    r = contrast.attention_contrast(attention, Q, K, V, [256] * 4, True, w["scale"])
    say(str(r))
    assert r["det_distinct_digests"] == 1
    assert r["f32_distinct_digests"] > 1
    assert 0 < r["f32_max_spread"] < 1e-5
    assert torch.equal(attention.det_attn_sharded(Q, K, V, [256] * 4, True, order=[2, 0, 3, 1]),
                       attention.det_attn(Q, K, V, True))


def test_vocab_splits_float32_vs_exact():
    from bitwise_deterministic_exact_pass1_amd import contrast, cross_entropy
    say("contrast: cross-entropy N=4096 V=128256 bf16, splits 1/2/4/8")
    x, t = W.ce_inputs()
    X, T = x.cuda(), t.cuda()
    del x
    r = contrast.ce_contrast(cross_entropy, X, T)
    say(str(r))
    assert all(n == 0 for n in r["det_flipped_losses"].values())
    assert r["f32_flipped_losses"][1] == 0 and r["f32_flipped_losses"][8] > 0
