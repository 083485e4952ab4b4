"""Pins of the oracle's byte accounting against the numbers the pages print.

Fixture: tests/golden/kv_size_closed_form.json (cited inside).
"""

import json
import os

import pytest

from oracle import pool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_size_closed_form.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN, encoding="utf-8") as f:
        return json.load(f)


def test_per_request_closed_form_matches_printed_value(golden):
    f = golden["factors"]
    nbytes = pool.kv_bytes_per_request(f["seq_len"], f["layers"], f["heads"], f["head_dim"],
                                       f["bytes_per_elem"])
    assert nbytes == 1_073_741_824  # the product itself, 2^30
    assert round(nbytes / 1e9, golden["printed_per_request_decimals"]) == \
        golden["printed_per_request_GB"]


def test_concurrent_requests_total_matches_printed_value(golden):
    f = golden["factors"]
    per = pool.kv_bytes_per_request(f["seq_len"], f["layers"], f["heads"], f["head_dim"],
                                    f["bytes_per_elem"])
    total = golden["printed_concurrent_requests"] * per
    assert round(total / 1e9, golden["printed_concurrent_decimals"]) == \
        golden["printed_concurrent_GB"]


def test_paged_pool_of_one_request_equals_closed_form(golden):
    """A pool holding exactly the ceil(2048/16) blocks of one request, in all
    32 layers, has the byte size the pages' closed form gives."""
    f = golden["factors"]
    block_size = 16
    n_blocks = -(-f["seq_len"] // block_size)
    nbytes = pool.pool_bytes(f["layers"], n_blocks, block_size, f["heads"], f["head_dim"], "f16")
    assert nbytes == pool.kv_bytes_per_request(f["seq_len"], f["layers"], f["heads"],
                                               f["head_dim"], f["bytes_per_elem"])


def test_fp8_halves_the_pool():
    a = pool.pool_bytes(1, 100, 16, 32, 128, "f16")
    b = pool.pool_bytes(1, 100, 16, 32, 128, "e4m3")
    c = pool.pool_bytes(1, 100, 16, 32, 128, "bf16")
    assert a == 2 * b == c


def test_element_layout_offsets():
    """The [L, 2, NB, Hkv, BS, D] view puts element (l, c, b, h, t, d) at the
    documented flat offset ((((l*2 + c)*NB + b)*Hkv + h)*BS + t)*D + d."""
    import numpy as np
    L, NB, H, BS, D = 2, 3, 2, 16, 4
    n = pool.pool_bytes(L, NB, BS, H, D, "f16")
    buf = np.zeros(n, dtype=np.uint8)
    view = pool.view_pool(buf, L, NB, BS, H, D, "f16")
    flat = buf.view(np.uint16)
    rng = np.random.default_rng(0)
    for _ in range(50):
        l, c, b, h, t, d = (int(rng.integers(0, s)) for s in (L, 2, NB, H, BS, D))
        view[...] = 0
        view[l, c, b, h, t, d] = 0xABCD
        off = ((((l * 2 + c) * NB + b) * H + h) * BS + t) * D + d
        assert flat[off] == 0xABCD and int(flat.sum()) == 0xABCD
