"""Pins for the oracle's block copies (host-memory KV tier): block sizes
against the pages' byte figures, and gather / scatter against numpy's own
indexing of the cache viewed as [num_blocks][block_bytes]."""
import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads


def test_block_bytes_match_the_pages():
    # gpt-oss-20b: 24,576 B per token over 12 full-attention layers in BF16 = 2,048 B per layer for
    # K and V (8 heads x 64 dims x 2 B x 2): one 16-token block of K is 16 KiB in BF16
    bf16 = oracle.block_bytes(oracle.KV_BF16, 8, 64)
    fp8 = oracle.block_bytes(oracle.KV_FP8, 8, 64)
    nv = oracle.block_bytes(oracle.KV_NVFP4, 8, 64)
    assert bf16 == 16 * 24576 // 12 // 2 == 16384
    assert fp8 * 2 == bf16                      # FP8 halves the payload
    assert nv * 8 == fp8 * 4.5                  # 4.5 bits per element
    assert nv == 8 * oracle.nvfp4_region_bytes(64, 16)


def test_gather_scatter_match_numpy_indexing():
    w = workloads.make("tiny", seed=51, seq_lens=[100, 40])
    kc, vc = oracle.new_caches(oracle.KV_FP8, w.num_blocks, w.Hkv, w.D, 16)
    oracle.cache_write(w.k, w.v, w.slot_mapping, kc, vc, oracle.KV_FP8, 0.02, 0.02)
    bb = oracle.block_bytes(oracle.KV_FP8, w.Hkv, w.D)
    ids = np.random.default_rng(3).permutation(w.num_blocks)[:5]
    got = oracle.gather_blocks(kc, ids, bb)
    assert np.array_equal(got, kc.view(np.uint8).reshape(w.num_blocks, bb)[ids])
    dst = np.zeros_like(kc)
    oracle.scatter_blocks(got, ids, bb, dst)
    want = np.zeros((w.num_blocks, bb), dtype=np.uint8)
    want[ids] = kc.view(np.uint8).reshape(w.num_blocks, bb)[ids]
    assert np.array_equal(dst.view(np.uint8).reshape(w.num_blocks, bb), want)


def test_round_trip_through_other_blocks_keeps_attention():
    # offload the blocks of a sequence, restore them into other physical blocks, re-point the block
    # table: attention is bit-identical
    w = workloads.make("tiny", seed=52, seq_lens=[64, 80])
    kc, vc = oracle.new_caches(oracle.KV_FP8, w.num_blocks + 9, w.Hkv, w.D, 16)
    oracle.cache_write(w.k, w.v, w.slot_mapping, kc, vc, oracle.KV_FP8, 0.02, 0.03)
    before = oracle.decode_attn(w.q, kc, vc, oracle.KV_FP8, w.block_tables, w.seq_lens, w.Hkv, 16, 0.02, 0.03, 0.125)
    bb = oracle.block_bytes(oracle.KV_FP8, w.Hkv, w.D)
    ids = w.block_tables[1, :5].numpy()
    host_k, host_v = oracle.gather_blocks(kc, ids, bb), oracle.gather_blocks(vc, ids, bb)
    new_ids = np.arange(w.num_blocks, w.num_blocks + 5, dtype=np.int32)
    oracle.scatter_blocks(host_k, new_ids, bb, kc)
    oracle.scatter_blocks(host_v, new_ids, bb, vc)
    bt = w.block_tables.clone()
    bt[1, :5] = torch.from_numpy(new_ids)
    after = oracle.decode_attn(w.q, kc, vc, oracle.KV_FP8, bt, w.seq_lens, w.Hkv, 16, 0.02, 0.03, 0.125)
    assert np.array_equal(before, after)


@pytest.mark.parametrize("fmt", [oracle.KV_BF16, oracle.KV_FP8, oracle.KV_NVFP4])
def test_threaded_cache_write_equals_the_serial_write(fmt):
    """Sharing the tokens out over threads by slot pair leaves every byte as the
    one-thread write leaves it: repeated slots (last write stays), skipped
    slots, neighbouring slots of one NVFP4 V byte, any slot order."""
    w = workloads.make("mixed64", seed=31, seq_lens=[300, 77, 150], shape=dict(Hq=4, Hkv=2, D=64))
    rng = np.random.default_rng(31)
    sm = w.slot_mapping.numpy().copy()
    sm[rng.choice(len(sm), 40, replace=False)] = -1                 # skipped
    dup = rng.choice(len(sm), 60, replace=False)
    sm[dup[:30]] = sm[dup[30:]]                                     # repeated slots
    outs = []
    for nthreads in (1, 3, 8):
        if fmt == oracle.KV_NVFP4:
            kc, vc = oracle.new_caches(fmt, w.num_blocks, w.Hkv, w.D, 16, fill=0x5A)
            oracle.nvfp4_cache_write(w.k, w.v, sm, kc, vc, 16, 0.01, 0.02, nthreads=nthreads)
        else:
            kc, vc = oracle.new_caches(fmt, w.num_blocks, w.Hkv, w.D, 16, fill=0x5A)
            oracle.cache_write(w.k, w.v, sm, kc, vc, fmt, 0.01, 0.02, nthreads=nthreads)
        outs.append((kc, vc))
    for kc, vc in outs[1:]:
        assert np.array_equal(kc, outs[0][0]) and np.array_equal(vc, outs[0][1])
