"""The packed weight layout of moe_grouped_ffn_packed (host logic, CPU only).

pack_weights must place W[r][k] of each [R][K] matrix at
((r/16) * (K/32) + k/32) * 512 + (((k%32)/8) * 16 + r%16) * 8 + k%8: blocks of
16 rows x 32 K values in which lane (row r%16, quarter (k%32)/8) of a 64-lane
wave finds its eight consecutive K values at 16 * lane bytes.
"""
import itertools

import pytest
import torch

import top_expert_routing_amd as moe


def _offset(r, k, K):
    return ((r // 16) * (K // 32) + k // 32) * 512 + (((k % 32) // 8) * 16 + r % 16) * 8 + k % 8


@pytest.mark.parametrize("E,R,K", [(1, 16, 32), (2, 32, 64), (3, 48, 96)])
def test_every_element_lands_at_its_offset(E, R, K):
    w = torch.arange(E * R * K, dtype=torch.float64).reshape(E, R, K)
    p = moe.pack_weights(w)
    assert p.shape == w.shape
    flat = p.reshape(E, R * K)
    for e, r, k in itertools.product(range(E), range(R), range(K)):
        assert flat[e, _offset(r, k, K)] == w[e, r, k]


def test_each_matrix_keeps_its_elements_and_place():
    w = torch.randn(4, 64, 128)
    p = moe.pack_weights(w)
    for e in range(4):
        assert torch.equal(torch.sort(p[e].flatten()).values, torch.sort(w[e].flatten()).values)


def test_a_block_is_one_contiguous_kilobyte_per_lane_order():
    # bf16: one 16 x 32 block = 1 KiB; lane L = 16 q + r reads bytes [16 L, 16 L + 16)
    w = torch.randn(1, 16, 32).to(torch.bfloat16)
    blk = moe.pack_weights(w).reshape(64, 8)
    for q, r in itertools.product(range(4), range(16)):
        assert torch.equal(blk[16 * q + r], w[0, r, 8 * q:8 * q + 8])


def test_shapes_that_do_not_tile_are_refused():
    with pytest.raises(ValueError):
        moe.pack_weights(torch.zeros(1, 24, 32))
    with pytest.raises(ValueError):
        moe.pack_weights(torch.zeros(1, 16, 48))


@pytest.mark.parametrize("E,R,K", [(1, 16, 64), (2, 32, 128)])
def test_fp8_codes_land_at_their_offsets(E, R, K):
    q = torch.randint(0, 256, (E, R, K), dtype=torch.uint8, generator=torch.Generator().manual_seed(R + K))
    flat = moe.pack_fp8_codes(q).reshape(E, R * K)
    for e, r, k in itertools.product(range(E), range(R), range(K)):
        off = ((r // 16) * (K // 64) + k // 64) * 1024 + (((k % 64) // 16) * 16 + r % 16) * 16 + k % 16
        assert flat[e, off] == q[e, r, k]


def test_fp8_shapes_that_do_not_tile_are_refused():
    with pytest.raises(ValueError):
        moe.pack_fp8_codes(torch.zeros(1, 16, 96, dtype=torch.uint8))
