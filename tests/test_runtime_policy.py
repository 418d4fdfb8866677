"""The decode batch's load policy, on the CPU with a stand-in cache.

Decode reads the pools with cacheable loads only when some block is shared between rows (forks, a
shared prompt), whose re-reads then hit in L2 and the Infinity Cache; when the sharing is a prefix of
the rows, only the tiles of that prefix are read cacheable and the rest streamed.  Every other batch,
FP8 or 16-bit, small or large, is streamed with the non-temporal hint.  `load_policy` overrides the rule.
"""
import types

import pytest

from paged_kv_cache_53_amd.runtime import DecodeBatch


def _batch(shared, quantised, tokens, policy="auto", prefix=0):
    cache = types.SimpleNamespace(has_shared_blocks=lambda: shared, quantised=quantised, n_kv_heads=8,
                                  head_dim=128)
    return types.SimpleNamespace(cache=cache, load_policy=policy, host_lens=[tokens], shared_prefix=prefix)


@pytest.mark.parametrize("quantised", [False, True])
@pytest.mark.parametrize("tokens", [16, 35_000, 1_200_000])
def test_shared_blocks_alone_select_cacheable_loads(quantised, tokens):
    assert DecodeBatch._load_args(_batch(True, quantised, tokens)) == {"shared_kv": True}
    # a small FP8 batch does not stay cacheable: streamed loads lost nothing after a read and
    # cacheable ones lost 48 % after a write
    assert DecodeBatch._load_args(_batch(False, quantised, tokens)) == {"shared_kv": False}


@pytest.mark.parametrize("shared", [False, True])
def test_policy_override(shared):
    assert DecodeBatch._load_args(_batch(shared, False, 100, "cached")) == {"shared_kv": True}
    assert DecodeBatch._load_args(_batch(shared, True, 100, "streamed")) == {}


def test_shared_prefix_is_read_cacheable_and_the_rest_streamed():
    b = _batch(True, False, 16000, prefix=4000)
    assert DecodeBatch._load_args(b) == {"shared_prefix_tokens": 4000}
    # shared blocks that are no prefix of the rows: every tile cacheable
    assert DecodeBatch._load_args(_batch(True, False, 100)) == {"shared_kv": True}
    assert DecodeBatch._load_args(_batch(False, False, 100)) == {"shared_kv": False}
    assert DecodeBatch._load_args(_batch(True, False, 100, "cached", prefix=64)) == {"shared_kv": True}
    assert DecodeBatch._load_args(_batch(True, False, 100, "streamed", prefix=64)) == {}


def test_shared_prefix_from_reference_counts():
    """The prefix is taken from the allocator: leading blocks of a row with more than one reference."""
    import numpy as np
    from paged_kv_cache_53_amd import Allocator
    a = Allocator(64, 16)
    a.alloc(9, 40)                       # a 40-token prompt: blocks 0, 1 full, block 2 with 8 tokens
    for c in (0, 1):
        a.fork(9, c, 32)                 # the children share its two full blocks
        a.alloc(c, 5)
    a.free(9)
    b = types.SimpleNamespace(cache=types.SimpleNamespace(allocator=a, block_size=16), S=2,
                              seq_ids=np.array([0, 1], dtype=np.int64), stride=4)
    assert DecodeBatch._find_shared_prefix(b) == 32
    a.alloc(2, 50)                       # a row of its own: no shared prefix
    b2 = types.SimpleNamespace(cache=types.SimpleNamespace(allocator=a, block_size=16), S=1,
                               seq_ids=np.array([2], dtype=np.int64), stride=4)
    assert DecodeBatch._find_shared_prefix(b2) == 0
