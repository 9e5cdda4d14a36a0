"""Token-budget step composer (host code, no GPU): the rule of "Chunked Prefill" (Ultralytics),
token-budget section, checked on the page's own setting and against a plain model of the rule on
random queues, plus its invariants."""
import random

import numpy as np
import pytest


def model(num_decode, remaining, budget, max_chunk):
    """Plain statement of the rule: one token per running decode first, then chunks in queue order."""
    dec = min(num_decode, budget)
    left = budget - dec
    chunks = []
    for r in remaining:
        c = min(r, left)
        if max_chunk > 0:
            c = min(c, max_chunk)
        chunks.append(c)
        left -= c
    return dec, chunks


def test_mixed_step_shape():
    """127 running decodes and a 32,768-token prompt under the 4,096-token budget of the vLLM
    configuration example in "第2章:推理引擎核心技术": the prompt gets the 3,969 tokens the decodes
    leave, and continues next step."""
    import paged_kv_cache_170_amd as pkv
    nd, ch = pkv.compose_step(127, [32768], 4096)
    assert nd == 127 and list(ch) == [4096 - 127]
    nd, ch = pkv.compose_step(127, [32768 - 3969], 4096)
    assert list(ch) == [3969]
    # With a 512-token chunk cap the second prompt picks up what the first leaves.
    nd, ch = pkv.compose_step(127, [300, 5000, 5000], 1000, max_chunk=512)
    assert nd == 127 and list(ch) == [300, 512, 61]


def test_random_queues_match_the_rule_and_invariants():
    import paged_kv_cache_170_amd as pkv
    rng = random.Random(0)
    for _ in range(500):
        nd_in = rng.randint(0, 300)
        rem = [rng.randint(1, 5000) for _ in range(rng.randint(0, 12))]
        budget = rng.randint(1, 9000)
        cap = rng.choice([0, 0, 256, 512, 2048])
        nd, ch = pkv.compose_step(nd_in, rem, budget, cap)
        assert (nd, list(ch)) == model(nd_in, rem, budget, cap)
        # Budget respected; decode tokens first; a chunk never exceeds what is left of its prompt.
        assert nd + int(np.sum(ch)) <= budget
        assert nd == min(nd_in, budget)
        assert all(0 <= c <= r for c, r in zip(ch, rem))
        # Nothing is left unused while work is waiting (up to the cap).
        if cap == 0 and nd + int(np.sum(ch)) < budget:
            assert list(ch) == rem


def test_bad_arguments():
    import paged_kv_cache_170_amd as pkv
    for args in ((-1, [5], 10), (1, [0], 10), (1, [5], 0)):
        with pytest.raises(pkv.PagedKVError) as e:
            pkv.compose_step(*args)
        assert e.value.status == pkv.INVALID_ARG
