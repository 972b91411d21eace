"""GPU parity of the packed variable-length forward (fa_fwd_varlen) against the
float64 oracle: ragged sequence lengths (empty, one row, tile multiples and
ragged tails), rows outside every sequence, grouped K/V heads, the max_seqlen
cut, and the packed training workload at full size on sampled rows."""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_56_amd as fa
import oracle
import workloads as W
from parity import TOL, assert_close, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def packed_inputs(lens, H, H_kv, d, dtype, seed, lead=0, tail=0, outliers=True):
    """Seeded packed inputs with `lead` rows before the first sequence and `tail`
    rows after the last (rows in no sequence)."""
    spec = W.SPECS["packed_causal_bf16"].with_shape(
        B=len(lens), H=H, H_kv=H_kv, d=d, dtype=dtype, seed=seed,
        outlier_frac=0.05 if outliers else 0.0)
    rng = np.random.default_rng(seed)
    T = lead + int(sum(lens)) + tail
    q = rng.standard_normal((H, T, d)).astype(np.float32)
    k = rng.standard_normal((H_kv, T, d)).astype(np.float32)
    v = rng.standard_normal((H_kv, T, d)).astype(np.float32)
    if outliers:
        idx = rng.choice(T, max(1, T // 20), replace=False)
        k[:, idx] *= np.float32(8.0)
    tdt = W.TORCH_STORAGE[dtype]
    qt, kt, vt = (torch.from_numpy(x).to(tdt) for x in (q, k, v))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32) + lead
    return spec, qt, kt, vt, cu


def run_packed(qt, kt, vt, cu, max_seqlen, scale, causal):
    q, k, v = (t.to(DEV) for t in (qt, kt, vt))
    H, T, d = q.shape
    o = torch.full((H, T, d), float("nan"), dtype=q.dtype, device=DEV)
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd_varlen(q, k, v, o, lse, torch.from_numpy(cu).to(DEV), max_seqlen, scale, causal)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


LENS = [
    [0, 1, 77, 300, 129, 256, 513],
    [1000],
    [128, 128, 0, 64, 65, 3],
    [31, 2, 700, 1, 255],
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_small(dtype, d, causal):
    for i, lens in enumerate(LENS):
        H, H_kv = (4, 2) if i % 2 else (2, 2)
        lead, tail = (5, 7) if i % 2 == 0 else (0, 0)
        seed = 12000 + 31 * i + d + 2 * causal + (dtype == "fp16")
        say(f"case packed dtype={dtype} d={d} causal={causal} lens={lens} H={H} H_kv={H_kv} "
            f"lead={lead} tail={tail} seed={seed}")
        spec, qt, kt, vt, cu = packed_inputs(lens, H, H_kv, d, dtype, seed, lead, tail)
        scale = 1.0 / math.sqrt(d)
        o, lse = run_packed(qt, kt, vt, cu, max(lens), scale, causal)
        qe, ke, ve = (t.double().numpy() for t in (qt, kt, vt))
        o_ref, lse_ref = oracle.attention_varlen(qe, ke, ve, cu, scale, causal)
        covered = ~np.isnan(lse_ref[0])
        # rows in no sequence are not written
        assert np.isnan(o[:, ~covered]).all() and np.isnan(lse[:, ~covered]).all()
        assert_close(o[:, covered], lse[:, covered], o_ref[:, covered], lse_ref[:, covered],
                     dtype, f"lens={lens}")


def test_packed_max_seqlen_cuts_and_clamped_bounds():
    lens = [300, 50, 700]
    spec, qt, kt, vt, cu = packed_inputs(lens, 2, 1, 128, "bf16", 12500, lead=3, tail=4)
    scale = 1.0 / math.sqrt(128)
    for max_seqlen in (256, 64, 1):
        say(f"case packed max_seqlen={max_seqlen}")
        o, lse = run_packed(qt, kt, vt, cu, max_seqlen, scale, True)
        qe, ke, ve = (t.double().numpy() for t in (qt, kt, vt))
        o_ref, lse_ref = oracle.attention_varlen(qe, ke, ve, cu, scale, True, max_seqlen)
        covered = ~np.isnan(lse_ref[0])
        assert np.isnan(lse[:, ~covered]).all()
        assert_close(o[:, covered], lse[:, covered], o_ref[:, covered], lse_ref[:, covered],
                     "bf16", f"max_seqlen={max_seqlen}")
    # a negative start is clamped to 0 and an end below its start gives an
    # empty sequence; an end past the packed rows is clamped to them
    T = qt.shape[1]
    qe, ke, ve = (t.double().numpy() for t in (qt, kt, vt))
    for cu2, segs in (([-7, 100, 40, 40], [(0, 100), (100, 0), (40, 0)]),
                      ([100, T + 500], [(100, T - 100)])):
        cu2 = np.array(cu2, dtype=np.int32)
        say(f"case packed clamped bounds cu={list(cu2)}")
        assert oracle.packed_segments(cu2, T) == segs
        o, lse = run_packed(qt, kt, vt, cu2, T, scale, False)
        o_ref, lse_ref = oracle.attention_varlen(qe, ke, ve, cu2, scale, False)
        covered = ~np.isnan(lse_ref[0])
        assert np.isnan(lse[:, ~covered]).all()
        assert_close(o[:, covered], lse[:, covered], o_ref[:, covered], lse_ref[:, covered],
                     "bf16", f"cu={list(cu2)}")


def test_packed_sequence_order_does_not_change_results():
    """Each sequence is computed the same wherever it sits in the packing:
    reversing the order of the sequences permutes the outputs bit for bit."""
    lens = [513, 1, 300, 1024, 77]
    spec, qt, kt, vt, cu = packed_inputs(lens, 4, 2, 128, "bf16", 12600)
    scale = 1.0 / math.sqrt(128)
    o, lse = run_packed(qt, kt, vt, cu, max(lens), scale, True)
    order = list(reversed(range(len(lens))))
    pieces = lambda x, axis: [np.take(x, np.arange(cu[b], cu[b + 1]), axis=axis) for b in order]
    q2, k2, v2 = (torch.from_numpy(np.concatenate(pieces(t.float().numpy(), 1), axis=1)).to(t.dtype)
                  for t in (qt, kt, vt))
    lens2 = [lens[b] for b in order]
    cu2 = np.concatenate([[0], np.cumsum(lens2)]).astype(np.int32)
    o2, lse2 = run_packed(q2, k2, v2, cu2, max(lens), scale, True)
    for pos, b in enumerate(order):
        a = slice(cu[b], cu[b + 1])
        c = slice(cu2[pos], cu2[pos + 1])
        assert np.array_equal(o[:, a], o2[:, c]) and np.array_equal(lse[:, a], lse2[:, c]), b


def test_packed_training_workload_sampled_rows():
    """The packed training batch at full size (16 sequences of 256..8192 rows,
    32 heads, d 128, causal) in the launch configuration the benchmark times,
    checked on rows computed one by one by the oracle."""
    spec = W.SPECS["packed_causal_bf16"]
    w = W.draw(spec)
    say(f"case packed workload {spec.name} T={w.q.shape[1]} lens={list(w.lengths)}")
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    o, lse = fa.fwd_varlen(q, k, v, cu, int(w.lengths.max()), scale=spec.scale, causal=True)
    torch.cuda.synchronize()
    o = o.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    qe, ke, ve = (t.double().numpy() for t in (w.q, w.k, w.v))
    rng = np.random.default_rng(5)
    worst = 0.0
    for b, n in enumerate(w.lengths):
        s0 = int(w.cu_seqlens[b])
        fixed = {0, 1, 63, 64, 127, 128, n // 2, n - 129, n - 1}
        rows = np.array(sorted({r for r in fixed if 0 <= r < n} |
                               set(int(r) for r in rng.choice(n, 8, replace=False))))
        for h in (0, 13, 31):
            o_ref, lse_ref = oracle.attention_varlen_rows(qe, ke, ve, w.cu_seqlens, spec.scale,
                                                          True, b, h, rows)
            err = np.abs(o[h, s0 + rows] - o_ref).max()
            dl = np.abs(lse[h, s0 + rows] - lse_ref).max()
            worst = max(worst, err)
            assert err <= TOL["bf16"]["max_o"], (b, h, err)
            assert dl <= TOL["bf16"]["lse"], (b, h, dl)
    say(f"  sampled rows max|dO|={worst:.3e}")
    assert np.isfinite(o).all() and np.isfinite(lse).all()
