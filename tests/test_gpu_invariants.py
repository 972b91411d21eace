"""Oracle-free checks of the GPU path that hold at any size, plus stream and
determinism behaviour."""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_56_amd as fa
import workloads as W
from parity import say, to_device

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def draw_small(name, **kw):
    return W.draw(W.SPECS[name].with_shape(**kw))


@pytest.mark.parametrize("name", ["long_causal_bf16", "long_causal_fp8", "encoder_padded_bf16"])
def test_bitwise_deterministic(name):
    """No atomics and a fixed reduction order: repeated launches agree bit for bit."""
    w = W.draw(W.SPECS[name])
    say(f"case determinism {name}")
    q, k, v, kl = to_device(w)
    outs = [fa.forward(q, k, v, w.spec.scale, w.spec.causal, kl, descale=w.descale)
            for _ in range(3)]
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0])
        assert torch.equal(lse, outs[0][1])


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32", "fp8"])
def test_causal_row_zero_is_v0_and_ones_give_ones(dtype):
    d = 128 if dtype == "fp8" else 64
    w = draw_small("decoder_causal_bf16", B=2, H=4, N=700, d=d, dtype=dtype, seed=91)
    say(f"case row0/ones dtype={dtype}")
    q, k, v, _ = to_device(w)
    o, lse = fa.forward(q, k, v, 0.125, True, None, descale=w.descale)
    v0 = v[:, :, 0].float() * w.descale[2]
    if dtype == "fp32":
        # exp2(c*s - c*m) with one FMA leaves the row's own weight within an
        # ulp or two of 1, and O = (p v) / p is then exact to a few ulps
        assert ((o[:, :, 0] - v0).abs() <= 1e-6 * v0.abs()).all()
    else:
        # the weight rounds to exactly 1 in 16-bit, so row 0 is V[0] exactly
        assert torch.equal(o[:, :, 0].float(), v0.to(o.dtype).float())
    ones = torch.ones_like(v)
    o1, _ = fa.forward(q, k, ones, 0.125, True, None, descale=(w.descale[0], w.descale[1], 1.0))
    torch.cuda.synchronize()
    # P's running sum and P V add the same values in different orders
    tol = 1e-5 if dtype == "fp32" else 1e-6
    assert (o1.float() - 1.0).abs().max().item() <= tol


def test_key_shift_leaves_o_unchanged_and_shifts_lse():
    """K -> K + 1 u^T adds scale * q_i.u to row i: O unchanged, LSE shifted (fp32)."""
    w = draw_small("single_head_fp32", B=2, H=2, N=333, d=128, seed=5)
    say("case key shift fp32")
    q, k, v, _ = to_device(w)
    u = torch.randn(128, generator=torch.Generator().manual_seed(3)).to(DEV)
    o, lse = fa.forward(q, k, v, 0.09, True)
    o2, lse2 = fa.forward(q, k + u, v, 0.09, True)
    torch.cuda.synchronize()
    assert (o - o2).abs().max().item() <= 2e-5
    shift = 0.09 * (q.double() @ u.double())
    assert ((lse2.double() - lse.double()) - shift).abs().max().item() <= 1e-4


def test_linearity_in_v_fp32():
    w = draw_small("single_head_fp32", B=1, H=3, N=257, d=64, seed=6)
    say("case linearity fp32")
    q, k, v, _ = to_device(w)
    v2 = torch.randn_like(v)
    a, _ = fa.forward(q, k, v, 0.125, False)
    b, _ = fa.forward(q, k, v2, 0.125, False)
    c, _ = fa.forward(q, k, v + v2, 0.125, False)
    torch.cuda.synchronize()
    assert (c - a - b).abs().max().item() <= 1e-5


def test_runs_on_a_side_stream_and_is_ordered():
    w = draw_small("decoder_causal_bf16", B=2, H=2, N=512, d=128, seed=8)
    say("case side stream")
    q, k, v, _ = to_device(w)
    ref, ref_lse = fa.forward(q, k, v, 0.1, True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q2 = q.clone()  # produced on the side stream, consumed on it in order
        o, lse = fa.forward(q2, k, v, 0.1, True, stream=s)
    s.synchronize()
    assert torch.equal(o, ref) and torch.equal(lse, ref_lse)


def test_outputs_untouched_on_argument_error():
    w = draw_small("decoder_causal_bf16", B=1, H=1, N=64, d=64, seed=9)
    q, k, v, _ = to_device(w)
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 1, 64), 7.0, device=DEV)
    with pytest.raises(fa.FaError):
        fa.fa_fwd(q, k, v, o, lse, -1.0)
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)


@pytest.mark.parametrize("dtype,N,causal", [("bf16", 300, True), ("fp16", 4200, True),
                                            ("fp8", 4096, False), ("fp32", 129, False)])
def test_grouped_heads_equal_repeated_heads_bit_for_bit(dtype, N, causal):
    """fa_fwd_gqa on [B,H_kv,N,d] K/V equals fa_fwd on the same K/V heads
    repeated to H: the same arithmetic on the same values, only addressed
    differently."""
    d = 128 if dtype == "fp8" else 64
    H, H_kv = 8, 2
    w = draw_small("decoder_causal_bf16", B=1, H=H, N=N, d=d, dtype=dtype, causal=causal,
                   seed=95, H_kv=H_kv)
    say(f"case grouped == repeated dtype={dtype} N={N} causal={causal}")
    q, k, v, _ = to_device(w)
    o_g, lse_g = fa.forward(q, k, v, 0.125, causal, None, descale=w.descale)
    rep = H // H_kv
    k_r = w.k.repeat_interleave(rep, dim=1).contiguous().to(DEV)
    v_r = w.v.repeat_interleave(rep, dim=1).contiguous().to(DEV)
    o_r, lse_r = fa.forward(q, k_r, v_r, 0.125, causal, None, descale=w.descale)
    torch.cuda.synchronize()
    assert torch.equal(o_g, o_r) and torch.equal(lse_g, lse_r)


@pytest.mark.parametrize("entry", ["fa_fwd_fp8", "fa_fwd_fp8_p8"])
@pytest.mark.parametrize("N,causal", [(300, True), (4096, False)])
def test_fp8_every_v_code_reaches_o_exactly(entry, N, causal):
    """key_len 1: every query row's only weight is 1 (on key 0), so O is V's row
    0 decoded with V's descale of 1, exactly. Row 0 of V holds every finite e4m3
    code (the two NaN codes replaced by 0) over the two batch entries, so each
    code's conversion to the P V operand is checked. N 300 causal runs the
    fp8 direct-to-LDS kernel, N 4096 the pipelined one (fa_fwd_fp8)."""
    B, H, d = 2, 1, 128
    g = torch.Generator().manual_seed(7)
    codes = torch.arange(256, dtype=torch.int32).reshape(B, d)
    codes[(codes & 0x7F) == 0x7F] = 0
    v8 = (torch.randint(0, 256, (B, H, N, d), generator=g, dtype=torch.int32) & 0x77)
    v8[:, 0, 0, :] = codes
    q = (torch.randn(B, H, N, d, generator=g) * 4).to(torch.float8_e4m3fn)
    k = (torch.randn(B, H, N, d, generator=g) * 4).to(torch.float8_e4m3fn)
    v = v8.to(torch.uint8).view(torch.float8_e4m3fn)
    expect = v[:, 0, 0, :].float()
    q, k, v = (t.to(DEV) for t in (q, k, v))
    o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=DEV)
    kl = torch.ones(B, dtype=torch.int32, device=DEV)
    say(f"case fp8 every code entry={entry} N={N} causal={causal}")
    getattr(fa, entry)(q, k, v, o, lse, 1.0 / math.sqrt(d), causal, kl)
    torch.cuda.synchronize()
    got = o.float().cpu()
    for b in range(B):
        assert torch.equal(got[b, 0], expect[b].expand(N, d)), f"batch {b}"
