"""The library without PyTorch: tests/c/decode_client (C++, raw HIP
allocations and a stream of its own, built by build()) calibrates, writes
the paged cache and runs decode attention through include/kvq.h alone.  Its
results are checked against the oracle: the amax values and scales exactly,
every cache byte bit for bit, and the attention within the path's tolerance.
The client runs as a child process (the test's own process does not touch
the GPU here)."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import assert_attention_close, gpu_or_skip, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c", "decode_client")


def bits16(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("kv,name,lens,shape,split", [
    (1, "gptoss65k", [3000, 517, 1, 0], dict(Hq=16, Hkv=2), 0),
    (1, "mixed64", [777, 2049], dict(Hq=16, Hkv=4, D=128), 256),
    (0, "agents126k", [1500, 90], dict(Hq=12, Hkv=2, D=256, calib_tokens=64), 128),
], ids=["fp8-d64", "fp8-d128", "bf16-d256"])
def test_c_client_matches_oracle(tmp_path, kv, name, lens, shape, split):
    gpu_or_skip()
    if not os.path.exists(CLIENT):
        pytest.fail(f"{CLIENT} is not built (build() builds it)")
    w = workloads.make(name, seed=141, seq_lens=lens, shape=shape)
    sm = float(np.float32(1.0 / np.sqrt(w.D)))
    d = str(tmp_path)
    with open(os.path.join(d, "params.txt"), "w") as f:
        f.write(f"{w.B} {w.Hq} {w.Hkv} {w.D} {w.T} {w.num_blocks} {w.block_tables.shape[1]} {w.max_seq_len} "
                f"{kv} {split} {sm:.9g}\n")
    bits16(w.q).tofile(os.path.join(d, "q.bin"))
    bits16(w.k).tofile(os.path.join(d, "k.bin"))
    bits16(w.v).tofile(os.path.join(d, "v.bin"))
    w.slot_mapping.numpy().astype(np.int64).tofile(os.path.join(d, "slots.bin"))
    w.block_tables.numpy().astype(np.int32).tofile(os.path.join(d, "bt.bin"))
    np.asarray(w.seq_lens, dtype=np.int32).tofile(os.path.join(d, "sl.bin"))
    say(f"c client: {name} kv={kv} lens={lens}")
    r = subprocess.run([CLIENT, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "decode_client: ok" in r.stdout, r.stdout + r.stderr

    amax_k, amax_v, ks, vs = (float.fromhex(x) for x in open(os.path.join(d, "scales.txt")).read().split())
    assert amax_k == oracle.amax_bf16(w.k) and amax_v == oracle.amax_bf16(w.v)
    if kv == 1:
        want = oracle.calibrate([amax_k, amax_v])
        assert (ks, vs) == (float(want[0]), float(want[1]))
        kvd = oracle.KV_FP8
    else:
        assert (ks, vs) == (1.0, 1.0)
        kvd = oracle.KV_BF16
    fill = 0xFF if kvd == oracle.KV_FP8 else 0xFFFF
    okc, ovc = oracle.new_caches(kvd, w.num_blocks, w.Hkv, w.D, 16, fill=fill)
    oracle.cache_write(w.k, w.v, w.slot_mapping, okc, ovc, kvd, ks, vs)
    kc = np.fromfile(os.path.join(d, "kc.bin"), dtype=np.uint8)
    vc = np.fromfile(os.path.join(d, "vc.bin"), dtype=np.uint8)
    assert np.array_equal(kc, okc.view(np.uint8).reshape(-1)) and np.array_equal(vc, ovc.view(np.uint8).reshape(-1))

    out = np.fromfile(os.path.join(d, "out.bin"), dtype=np.float32).reshape(w.B, w.Hq, w.D)
    ref = oracle.decode_attn(w.q, okc, ovc, kvd, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs, sm, nthreads=8)
    assert_attention_close(out, ref, f"c client {name}")
