"""GPU parity: libfa's output against the float64 oracle on seeded inputs.

Small shapes (full oracle) sweep every dtype, both head sizes, causal and
padding masks, ragged N and the degenerate cases; the five named workloads are
checked at their full sizes in the launch configuration the benchmark times,
against the full oracle where it finishes in seconds and against oracle rows
computed one by one otherwise.
"""
import math
import time

import numpy as np
import pytest
import torch

import exact_io_aware_56_amd as fa
import oracle
import workloads as W
from parity import assert_close, full_oracle, run, sampled_rows, say, to_device

pytestmark = pytest.mark.gpu

BASE = {"bf16": "decoder_causal_bf16", "fp16": "decoder_causal_bf16",
        "fp32": "single_head_fp32", "fp8": "long_causal_fp8"}


def small_spec(dtype, d, N, causal, padded, B=2, H=3, seed=0, outliers=None):
    """Small workload of the dtype's family. 16-bit and fp8 sweeps include 5%
    outlier keys (x8); fp32 keeps unit-variance inputs, the distribution its
    1e-5 bound is stated for (see test_fp32_outlier_keys for the rest)."""
    s = W.SPECS[BASE[dtype]]
    if outliers is None:
        outliers = dtype != "fp32"
    return s.with_shape(B=B, H=H, N=N, d=d, dtype=dtype, causal=causal,
                        scale=1.0 / math.sqrt(d),
                        key_len_range=(max(0, N // 3), N) if padded else None,
                        outlier_frac=0.05 if (N >= 40 and outliers) else 0.0, seed=seed)


SWEEP_N = [1, 2, 3, 15, 16, 17, 31, 33, 63, 64, 65, 127, 128, 129, 200, 257, 300]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp8", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_small_shape_sweep(dtype, d, causal):
    for i, N in enumerate(SWEEP_N):
        for padded in (False, True):
            spec = small_spec(dtype, d, N, causal, padded, seed=7000 + 17 * i + padded)
            say(f"case dtype={dtype} d={d} causal={causal} N={N} padded={padded} seed={spec.seed}")
            w = W.draw(spec)
            o, lse = run(w)
            o_ref, lse_ref = full_oracle(w)
            assert_close(o, lse, o_ref, lse_ref, dtype, f"N={N} padded={padded}")


# Sequences from 4096 keys on run the pipelined 16-bit kernel (256 query rows
# per workgroup); these cover it with one or two heads, so the full oracle
# stays cheap: exact multiples of its tiles, ragged ends, padding and causal
# masks, both head sizes.
LONG_N = [(4096, False), (4161, True), (4416, False)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_long_sequence_sweep(dtype, d, causal):
    for i, (N, padded) in enumerate(LONG_N):
        spec = small_spec(dtype, d, N, causal, padded, B=2 if padded else 1, H=1,
                          seed=9100 + 13 * i + 2 * d + causal)
        say(f"case long dtype={dtype} d={d} causal={causal} N={N} padded={padded} seed={spec.seed}")
        w = W.draw(spec)
        o, lse = run(w)
        o_ref, lse_ref = full_oracle(w)
        assert_close(o, lse, o_ref, lse_ref, dtype, f"N={N} padded={padded}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_long_sequence_growing_and_degenerate(dtype):
    """The pipelined kernel's lazy reference maximum under keys that grow
    along the sequence (many reference moves), and degenerate key lengths."""
    spec = small_spec(dtype, 128, 4224, True, True, B=1, H=2, seed=9300, outliers=False)
    w = W.draw(spec)
    grow = torch.linspace(0.2, 40.0, spec.N).reshape(1, 1, spec.N, 1)  # logits reach ~100
    w.k = (w.k.to(torch.float32) * grow).to(w.k.dtype)
    say(f"case long growing logits dtype={dtype}")
    o, lse = run(w)
    o_ref, lse_ref = full_oracle(w)
    assert_close(o, lse, o_ref, lse_ref, dtype, "long growing")

    spec = small_spec(dtype, 64, 4100, True, False, B=5, H=1, seed=9301)
    w = W.draw(spec)
    w.key_len = np.array([0, 1, -7, 10000, 4033], dtype=np.int32)
    say(f"case long degenerate key_len dtype={dtype}")
    o, lse = run(w)
    o_ref, lse_ref = full_oracle(w)
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf) and np.all(lse[2] == -np.inf)
    assert_close(o, lse, o_ref, lse_ref, dtype, "long degenerate")


def test_fp32_outlier_keys():
    """fp32 with x8 outlier keys: the logits reach ~30 and a 128-term fp32 dot
    product carries ~1e-6 relative rounding, so exp(logit) is off by up to
    ~3e-6 relative. The bar here is 4e-5 (O values are O(1))."""
    for i, (N, causal) in enumerate([(300, False), (257, True)]):
        spec = small_spec("fp32", 128, N, causal, False, seed=8100 + i, outliers=True)
        say(f"case fp32 outliers N={N} causal={causal} seed={spec.seed}")
        w = W.draw(spec)
        o, lse = run(w)
        o_ref, lse_ref = full_oracle(w)
        from parity import errors
        mx, mean, dl, same_inf = errors(o, lse, o_ref, lse_ref, True)
        say(f"  max|dO|={mx:.3e} mean|dO|={mean:.3e} max|dLSE|={dl:.3e}")
        assert same_inf and mx <= 4e-5 and mean <= 1e-6 and dl <= 1e-5


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("fp16", 64), ("fp16", 128),
                                     ("fp8", 128), ("fp32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_running_max_keeps_growing(dtype, d, causal):
    """Keys scaled up along the sequence so every key tile raises the row
    maxima, by small and by very large steps: the running-max correction
    (and its threshold, or the lazy reference's sum check) must reproduce the
    exact softmax. Causal 16-bit inputs at this length take the direct-to-LDS
    kernel, the others the pipelined or register-staged ones."""
    spec = small_spec(dtype, d, 700, causal, True, B=2, H=2, seed=8300 + causal + d, outliers=False)
    w = W.draw(spec)
    grow = torch.linspace(0.2, 6.0, spec.N).reshape(1, 1, spec.N, 1)
    if dtype == "fp8":
        k = (w.k.to(torch.float32) * grow).clamp(-448, 448)
        w.k = k.to(torch.float8_e4m3fn)
    else:
        w.k = (w.k.to(torch.float32) * grow).to(w.k.dtype)
    say(f"case growing logits dtype={dtype} causal={causal}")
    o, lse = run(w)
    o_ref, lse_ref = full_oracle(w)
    if dtype == "fp32":
        # logits up to ~40: the fp32 dot-product bar of test_fp32_outlier_keys
        from parity import errors
        mx, mean, dl, same_inf = errors(o, lse, o_ref, lse_ref, True)
        say(f"  max|dO|={mx:.3e} mean|dO|={mean:.3e} max|dLSE|={dl:.3e}")
        assert same_inf and mx <= 4e-5 and mean <= 1e-6 and dl <= 1e-5
    else:
        assert_close(o, lse, o_ref, lse_ref, dtype, "growing")


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp32", "fp16"])
def test_degenerate_key_lengths(dtype):
    """key_len 0 (no key: O = 0, LSE = -inf), 1, negative and above N (clamped)."""
    spec = small_spec(dtype, 128 if dtype == "fp8" else 64, 150, True, False, B=5, H=2,
                      seed=31)
    w = W.draw(spec)
    w.key_len = np.array([0, 1, -7, 1000, 77], dtype=np.int32)
    say(f"case degenerate key_len dtype={dtype}")
    o, lse = run(w)
    o_ref, lse_ref = full_oracle(w)
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf) and np.all(lse[2] == -np.inf)
    assert_close(o, lse, o_ref, lse_ref, dtype, "degenerate")


@pytest.mark.parametrize("name", ["single_head_fp32", "encoder_padded_bf16",
                                  "decoder_causal_bf16"])
def test_named_workload_full_oracle(name):
    w = W.draw(W.SPECS[name])
    say(f"case {name} full oracle seed={w.spec.seed}")
    o, lse = run(w)
    t0 = time.perf_counter()
    o_ref, lse_ref = full_oracle(w)
    say(f"  {name}: oracle {time.perf_counter() - t0:.2f} s")
    assert_close(o, lse, o_ref, lse_ref, w.spec.dtype, name)


@pytest.mark.parametrize("name", ["long_causal_bf16", "long_causal_fp8", "long_causal_grouped_bf16",
                                  "long_causal_d256_bf16"])
def test_named_workload_sampled_rows(name):
    """Full-size long-context workloads: every head, sampled rows (tile edges,
    the outlier keys' own rows, random rows) against the oracle row by row."""
    w = W.draw(W.SPECS[name])
    s = w.spec
    say(f"case {name} sampled rows seed={s.seed}")
    o, lse = run(w)
    q, k, v = w.exact()
    rng = np.random.default_rng(s.seed + 1)
    errs_o, errs_l = [], []
    for b in range(s.B):
        for h in range(s.H):
            g = h // (s.H // s.kv_heads)
            extra = None if w.outlier_rows is None else w.outlier_rows[b, g][:8]
            rows = sampled_rows(s, rng, per_head=24, extra=extra)
            o_ref, lse_ref = oracle.attention_rows(q, k, v, s.scale, s.causal,
                                                   w.key_len_or_none(), b, h, rows)
            errs_o.append(o[b, h, rows] - o_ref)
            errs_l.append(lse[b, h, rows] - lse_ref)
    eo = np.abs(np.concatenate(errs_o))
    el = np.abs(np.concatenate(errs_l))
    from parity import TOL
    t = TOL[s.dtype]
    say(f"  {name}: rows={eo.shape[0]} max|dO|={eo.max():.3e} mean|dO|={eo.mean():.3e} "
        f"max|dLSE|={el.max():.3e}")
    assert np.all(np.isfinite(o))
    assert eo.max() <= t["max_o"] and eo.mean() <= t["mean_o"] and el.max() <= t["lse"]


# Grouped K/V heads (fa_fwd_gqa): every kernel family, multi-query (H_kv = 1),
# grouped and ungrouped through the grouped entry point, both masks.
GROUPED = [  # dtype, d, N, causal, padded, H, H_kv
    ("bf16", 64, 300, True, False, 8, 2), ("bf16", 128, 129, False, True, 6, 3),
    ("fp16", 128, 257, True, True, 4, 1), ("fp16", 64, 65, False, False, 4, 4),
    ("fp32", 64, 200, True, True, 6, 2), ("fp32", 128, 33, False, False, 3, 1),
    ("fp8", 128, 300, True, False, 8, 2), ("fp8", 64, 127, False, True, 4, 1),
    # sequences long enough for the pipelined kernel
    ("bf16", 128, 4161, True, False, 4, 1), ("fp16", 64, 4096, False, True, 4, 2),
    ("fp8", 128, 4160, True, True, 2, 1),
]


@pytest.mark.parametrize("dtype,d,N,causal,padded,H,H_kv", GROUPED)
def test_grouped_kv_heads(dtype, d, N, causal, padded, H, H_kv):
    spec = small_spec(dtype, d, N, causal, padded, B=2 if N < 1000 else 1, H=H,
                      seed=9500 + N + H_kv).with_shape(H_kv=H_kv)
    say(f"case grouped dtype={dtype} d={d} N={N} causal={causal} padded={padded} "
        f"H={H} H_kv={H_kv} seed={spec.seed}")
    w = W.draw(spec)
    o, lse = run(w)
    o_ref, lse_ref = full_oracle(w)
    assert_close(o, lse, o_ref, lse_ref, dtype, f"H={H} H_kv={H_kv}")


# Head dimension 256 (16-bit inputs): two workgroups per query tile, one per
# column half of O; ragged tiles, padding, grouped heads and a longer sequence.
D256 = [(1, False, 2, 2, 2), (33, True, 2, 3, 3), (127, False, 1, 4, 2), (300, True, 2, 2, 1),
        (1000, False, 1, 2, 2),
        # long enough for the pipelined kernel's column slices with a causal mask
        (4160, False, 1, 2, 1), (4097, True, 1, 2, 2)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dim_256(dtype, causal):
    for i, (N, padded, B, H, H_kv) in enumerate(D256):
        spec = small_spec(dtype, 256, N, causal, padded, B=B, H=H,
                          seed=9700 + 11 * i + causal).with_shape(H_kv=H_kv)
        say(f"case d256 dtype={dtype} causal={causal} N={N} padded={padded} H={H}/{H_kv} "
            f"seed={spec.seed}")
        w = W.draw(spec)
        o, lse = run(w)
        o_ref, lse_ref = full_oracle(w)
        assert_close(o, lse, o_ref, lse_ref, dtype, f"d256 N={N}")


# Windows over sequences long enough for the pipelined kernel (causal N >= 4096;
# every non-causal length takes it): bands narrower and wider than its 256-row
# query tiles, a band of zero width, a two-sided band, padding and grouped heads.
LONG_WINDOWS = [  # causal, (left, right), N, padded, H_kv
    (True, (100, -1), 4160, False, 2), (True, (1000, -1), 4097, True, 1), (True, (0, -1), 4096, False, 2),
    (True, (300, 5), 4160, True, 2), (False, (130, 0), 4160, False, 1), (False, (40, 700), 4100, True, 2)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
def test_sliding_window_long(dtype, d):
    for i, (causal, window, N, padded, H_kv) in enumerate(LONG_WINDOWS):
        spec = small_spec(dtype, d, N, causal, padded, B=1, H=2,
                          seed=9950 + 7 * i + d).with_shape(H_kv=H_kv)
        say(f"case long window dtype={dtype} d={d} causal={causal} window={window} N={N} "
            f"padded={padded} H_kv={H_kv} seed={spec.seed}")
        w = W.draw(spec)
        q, k, v, kl = to_device(w)
        o, lse = fa.fwd(q, k, v, scale=spec.scale, causal=causal, key_len=kl, window=window)
        torch.cuda.synchronize()
        qe, ke, ve = w.exact()
        o_ref, lse_ref = oracle.attention_forward(qe, ke, ve, spec.scale, causal,
                                                  w.key_len_or_none(), window=window)
        assert_close(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, lse_ref,
                     dtype, f"window={window} N={N}")


def test_window_workload_sampled_rows():
    """The full-size sliding-window workload: every head, sampled rows
    (tile edges, band edges, random rows) against the oracle row by row."""
    w = W.draw(W.SPECS["long_causal_window_bf16"])
    s = w.spec
    window = (s.window_left, -1)
    say(f"case long_causal_window_bf16 sampled rows seed={s.seed}")
    q, k, v, kl = to_device(w)
    o, lse = fa.fwd(q, k, v, scale=s.scale, causal=s.causal, key_len=kl, window=window)
    torch.cuda.synchronize()
    o, lse = o.double().cpu().numpy(), lse.double().cpu().numpy()
    qe, ke, ve = w.exact()
    rng = np.random.default_rng(s.seed + 1)
    errs_o, errs_l = [], []
    for h in range(s.H):
        edges = [s.window_left - 1, s.window_left, s.window_left + 1, 255, 256, 257, s.N - 1]
        rows = sorted(set(edges) | set(rng.integers(0, s.N, 16).tolist()))
        o_ref, lse_ref = oracle.attention_rows(qe, ke, ve, s.scale, s.causal, w.key_len_or_none(),
                                               0, h, rows, window=window)
        errs_o.append(o[0, h, rows] - o_ref)
        errs_l.append(lse[0, h, rows] - lse_ref)
    eo = np.abs(np.concatenate(errs_o))
    el = np.abs(np.concatenate(errs_l))
    from parity import TOL
    t = TOL[s.dtype]
    say(f"  window workload: rows={eo.shape[0]} max|dO|={eo.max():.3e} mean|dO|={eo.mean():.3e} "
        f"max|dLSE|={el.max():.3e}")
    assert np.all(np.isfinite(o))
    assert eo.max() <= t["max_o"] and eo.mean() <= t["mean_o"] and el.max() <= t["lse"]


# Sliding windows (fa_fwd_window): bands on either side, with and without the
# causal mask, ragged lengths, padding and grouped heads.
WINDOWS = [  # causal, (left, right)
    (True, (0, -1)), (True, (63, -1)), (True, (100, -1)), (False, (5, 7)), (False, (-1, 3)),
    (False, (130, 0)), (True, (1000, -1))]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
def test_sliding_window(dtype, d):
    for i, (causal, window) in enumerate(WINDOWS):
        for N, padded in ((1, False), (65, True), (300, False), (1000, True)):
            H_kv = 1 if i % 2 else 2
            spec = small_spec(dtype, d, N, causal, padded, B=2, H=2,
                              seed=9900 + 7 * i + N + d).with_shape(H_kv=H_kv)
            say(f"case window dtype={dtype} d={d} causal={causal} window={window} N={N} "
                f"padded={padded} H_kv={H_kv} seed={spec.seed}")
            w = W.draw(spec)
            q, k, v, kl = to_device(w)
            o, lse = fa.fwd(q, k, v, scale=spec.scale, causal=causal, key_len=kl, window=window)
            torch.cuda.synchronize()
            qe, ke, ve = w.exact()
            o_ref, lse_ref = oracle.attention_forward(qe, ke, ve, spec.scale, causal,
                                                      w.key_len_or_none(), window=window)
            assert_close(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, lse_ref,
                         dtype, f"window={window} N={N}")
