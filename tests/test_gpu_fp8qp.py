"""GPU parity for the FP8 Q and P variant against the oracle's definition
(E4M3 Q with a calibrated q_scale, power-of-two softmax reference, P codes
E4M3(448 * 2^(x - R)), quantized weights in numerator and denominator).

The variant quantizes the softmax weights, so a score error of any size can
move a weight across an E4M3 rounding midpoint, and a one-pass kernel
quantizes each weight against the running power-of-two reference it holds,
which rounds the smallest weights on another grid.  Its tolerance therefore
comes from the definition, not from the kernel: the oracle's
kvqo_decode_attn_fp8qp_tol bounds every output of an implementation whose
scores and weighted sums are accurate to eps = 2^-10 of the sum of their
terms' magnitudes (an assumption: the matrix-core ISA states no rounding for
its FP8 dot steps) and whose references are powers of two up to the final
one.  Each output element must lie within that tolerance of the definition's
fp64 result.  Also: bf16 = RNE(fp32), multi-query, windows, every
column-tile count, and the variant's distance from the exact FP8 path."""
import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import Setup, assert_attention_close, gpu_or_skip, gpu_calibrate, kvq, say

pytestmark = pytest.mark.gpu

EPS = 2.0 ** -10   # assumed accuracy of the FP8 dot steps and sums (see the module docstring)

CASES = [
    # name, seed, seq_lens, shape, q_len, window, split_tokens
    ("gptoss65k", 81, [1000, 4097, 70], dict(Hq=16, Hkv=2), 1, 0, 0),
    ("gptoss65k", 82, [700, 2100, 5], dict(Hq=16, Hkv=2), 4, 0, 128),
    ("gptoss65k", 83, [2049, 300], dict(Hq=16, Hkv=2), 8, 0, 64),
    ("mixed64", 84, [777, 1500], dict(Hq=16, Hkv=4, D=128), 2, 0, 256),
    ("agents126k", 85, [1200, 97], dict(Hq=12, Hkv=2, D=256, calib_tokens=256), 1, 100, 64),
]


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


def run_qp(K, s, q, qs, split, window=0, dtype=torch.float32):
    w = s.w
    out = torch.empty(w.B, q.shape[1], w.Hq, w.D, dtype=dtype, device="cuda")
    ws = K.new_workspace_mq(w.B, q.shape[1], w.Hq, w.Hkv, w.D, w.max_seq_len, split, window=window)
    K.kvq_paged_decode_attn_fp8qp(q.cuda(), s.kc, s.vc, s.bt, s.sl, w.max_seq_len, w.Hkv, qs, s.ks, s.vs,
                                  s.sm_scale, out, ws, split_tokens=split, window=window)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fp8qp_matches_oracle(K, case):
    name, seed, lens, shape, q_len, window, split = CASES[case]
    w = workloads.make(name, seed=seed, seq_lens=lens, shape=shape)
    say(f"fp8qp case {case}: lens={lens} Hq={w.Hq} Hkv={w.Hkv} D={w.D} q_len={q_len} W={window} split={split}")
    s = Setup(w, 1)
    q = workloads.mq_queries(w, q_len, seed=seed)
    qs = gpu_calibrate(K, q.cuda())
    kc, vc = s.oracle_caches()
    ref = oracle.decode_attn_fp8qp(q, kc, vc, w.block_tables, w.seq_lens, w.Hkv, 16, qs, s.ks, s.vs, s.sm_scale,
                                   nthreads=8, window=window)
    tol, n_open = oracle.decode_attn_fp8qp_tol(q, kc, vc, w.block_tables, w.seq_lens, w.Hkv, 16, qs, s.ks, s.vs,
                                               s.sm_scale, EPS, window=window)
    out32 = run_qp(K, s, q, qs, split, window)
    got = out32.cpu().numpy()
    n_tok = sum(min(L, window) if window else L for L in w.seq_lens) * q_len * w.Hq
    err = np.abs(got - ref)
    frac = err / np.maximum(tol, 1e-300)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    say(f"  fp8qp case={case}: max |got - def| {err.max():.2e}, max of |got - def| / tol {frac.max():.3f}, "
        f"tol median {np.median(tol):.2e} max {tol.max():.2e}, open codes {n_open} of {n_tok} tokens, "
        f"rel L2 vs definition {rel:.2e}")
    assert np.isfinite(got).all() and np.isfinite(tol).all()
    assert (err <= tol).all(), float(frac.max())
    out16 = run_qp(K, s, q, qs, split, window, torch.bfloat16)
    assert torch.equal(out16.cpu().view(torch.int16), out32.cpu().to(torch.bfloat16).view(torch.int16))


def test_fp8qp_distance_from_the_exact_path(K):
    w = workloads.make("gptoss65k", seed=86, seq_lens=[3000, 900], shape=dict(Hq=16, Hkv=2))
    s = Setup(w, 1)
    q = workloads.mq_queries(w, 2, seed=1)
    qp = run_qp(K, s, q, gpu_calibrate(K, q.cuda()), 0)
    out = torch.empty_like(qp)
    ws = K.new_workspace_mq(w.B, 2, w.Hq, w.Hkv, w.D, w.max_seq_len)
    K.kvq_paged_decode_attn_mq(q.cuda(), s.kc, s.vc, 1, s.bt, s.sl, w.max_seq_len, w.Hkv, s.ks, s.vs, s.sm_scale,
                               out, ws)
    torch.cuda.synchronize()
    rel = float((qp - out).norm() / out.norm())
    say(f"  fp8qp vs exact FP8 path: rel L2 {rel:.3e}")
    assert rel < 0.15
