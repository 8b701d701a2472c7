"""Fixtures under tests/golden: the oracle against its stored regression
outputs, and the serving defaults against the constants the deployment page
prints (the xdnf.cn page "为什么 MoE 稀疏激活在长上下文下反而更吃显存", section 3)."""
import inspect
import json
import os
import sys

import numpy as np

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, GOLDEN)
import make_golden  # noqa: E402


def test_oracle_matches_stored_tiny_outputs():
    ref = json.load(open(os.path.join(GOLDEN, "oracle_tiny.json")))
    q, k, v, x = make_golden.tiny_inputs()
    out, S, _ = O.forward(q, k, v, x, gated=True)
    yn, _, zn = O.forward(q + 1.0, k + 1.0, v, normalized=True)
    for got, key in ((out, "gated_out"), (S, "state"), (yn, "normalized_y"), (zn, "normalized_z")):
        want = np.array(ref[key])
        assert got.shape == want.shape, key
        assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max()), key


def test_serving_defaults_follow_the_page():
    cfg = json.load(open(os.path.join(GOLDEN, "pages_serving_config.json")))
    from linear_attention_long_amd import api, serving
    budget = cfg["max_num_batched_tokens"]
    assert inspect.signature(api.la_schedule_step).parameters["max_batched_tokens"].default == budget
    assert inspect.signature(serving.run).parameters["max_batched_tokens"].default == budget
    assert cfg["enable_chunked_prefill"] is True
    # the page's block size and every pad size are accepted block sizes of the
    # library (the plan reports the block a call runs with)
    from linear_attention_long_amd import _lib
    for b in [cfg["lightning_attention_block_size"]] + cfg["tail_pad_options"]:
        p = _lib.plan(False, 1, 1000, 1000, 8, 128, _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_F32,
                      _lib.options(block_size=b))
        assert p.block_size == b
