"""The decode batch's load policy, on the CPU with a stand-in cache.

Decode reads the pools with cacheable loads only when some block is shared between rows (forks, a
shared prompt), whose re-reads then hit in L2 and the Infinity Cache; every other batch, FP8 or
16-bit, small or large, is streamed with the non-temporal hint.  `load_policy` overrides the rule.
"""
import types

import pytest

from paged_kv_cache_53_amd.runtime import DecodeBatch


def _batch(shared, quantised, tokens, policy="auto"):
    cache = types.SimpleNamespace(has_shared_blocks=lambda: shared, quantised=quantised, n_kv_heads=8,
                                  head_dim=128)
    return types.SimpleNamespace(cache=cache, load_policy=policy, host_lens=[tokens])


@pytest.mark.parametrize("quantised", [False, True])
@pytest.mark.parametrize("tokens", [16, 35_000, 1_200_000])
def test_shared_blocks_alone_select_cacheable_loads(quantised, tokens):
    assert DecodeBatch._keep_cached(_batch(True, quantised, tokens)) is True
    # a small FP8 batch no longer stays cacheable: streamed loads lost nothing after a read and
    # cacheable ones lost 48 % after a write
    assert DecodeBatch._keep_cached(_batch(False, quantised, tokens)) is False


@pytest.mark.parametrize("shared", [False, True])
def test_policy_override(shared):
    assert DecodeBatch._keep_cached(_batch(shared, False, 100, "cached")) is True
    assert DecodeBatch._keep_cached(_batch(shared, True, 100, "streamed")) is False
