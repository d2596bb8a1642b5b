"""Parity at the longest sequence the library accepts: T d_v x 2 bytes just
under 2^31 for bf16 tokens, so T = 8,388,607 at d_v = 128 (one head; the
32-bit offsets of the kernels' buffer stores are at their limit).  Covered:
the pipelined GDN kernel, the single-pass add-rule kernel, the two-kernel KDA
path, the one-pass normalised kernel and Gated DeltaProduct over its virtual
sequence read in place; and one decode step over a state of 2^32 elements.

The decay is strong (a_t <= e^-0.7 < 0.5 per token, per channel for KDA), and
with unit-norm keys and beta in (0, 1) the delta-rule factor (I - beta k k^T)
does not grow the state, so a token's output and the final state depend on
what lies more than W tokens back only up to 0.5^W of their size.  The oracle
therefore checks the first tokens from the start, and the last ones and two
runs in the middle (one across the output row at byte offset 2^30) each from a
window of W earlier tokens started at the zero state (W = 160: 0.5^160 is far
below the bf16 tolerance)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, host, note, rel_l2

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DV = 128
T_MAX = (2 ** 31 - 1) // (DV * 2)          # 8,388,607
HEAD, WIN, TAIL = 200, 160, 96             # checked prefix, warm-up window, checked tail


def draw(shapes, seed, unit=(), positive=()):
    """Seeded device draws in bf16: N(0,1), unit-norm rows for the names in
    ``unit``, elu + 1 of N(0,1) for ``positive``, log-gates -0.7 - 0.5 U(0,1)
    for 'g' and sigmoid(N(0,1)) for 'beta'."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    out = {}
    for name, shape in shapes.items():
        if name == "g":
            x = -0.7 - 0.5 * torch.rand(shape, generator=gen, device="cuda")
        elif name == "beta":
            x = torch.sigmoid(torch.randn(shape, generator=gen, device="cuda"))
        else:
            x = torch.randn(shape, generator=gen, device="cuda")
            if name in unit:
                x = x / x.norm(dim=-1, keepdim=True)
            if name in positive:
                x = torch.nn.functional.elu(x) + 1.0
        out[name] = x.to(torch.bfloat16)
        del x
    return out


def piece(x, sl):
    return {n: host(t[:, :, sl]) for n, t in x.items()}


def check_ends(name, T, outs, ref):
    """outs: (o [1,1,T,dv] on the device, final states ...); ref(sl) -> the
    oracle's (o, final states ...) for the tokens in slice sl from zero."""
    o = outs[0]
    o_head = ref(slice(0, HEAD))[0]
    e_head = rel_l2(host(o[:, :, :HEAD]), o_head)
    tail = ref(slice(T - WIN - TAIL, T))
    e_tail = rel_l2(host(o[:, :, T - TAIL:]), tail[0][:, :, WIN:])
    e_states = [rel_l2(host(s), sr) for s, sr in zip(outs[1:], tail[1:])]
    # windows inside the sequence: one a third of the way in, and one whose
    # checked tokens straddle the output row where the byte offset passes 2^30
    e_mid = []
    for c in (T // 3, (1 << 30) // (DV * 2)):
        t0 = c - TAIL // 2
        win = ref(slice(t0 - WIN, t0 + TAIL))
        e_mid.append(rel_l2(host(o[:, :, t0:t0 + TAIL]), win[0][:, :, WIN:]))
    note(f"[max] {name} T={T}: rel L2 first {HEAD} {e_head:.3e}, last {TAIL} {e_tail:.3e}, "
         f"middle windows {', '.join(f'{e:.3e}' for e in e_mid)}, "
         f"final states {', '.join(f'{e:.3e}' for e in e_states)}")
    assert max([e_head, e_tail] + e_mid + e_states) <= TOL["bf16"]


@pytest.mark.timeout(600)
def test_gdn_pipelined_max_length():
    import gated_delta_rule_27_amd as la
    T = T_MAX
    x = draw({"q": (1, 1, T, 128), "k": (1, 1, T, 128), "v": (1, 1, T, DV), "g": (1, 1, T),
              "beta": (1, 1, T)}, seed=401, unit=("q", "k"))
    o, s = la.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None, rule="delta", gate="scalar")
    torch.cuda.synchronize()

    def ref(sl):
        w = piece(x, sl)
        return oracle.recurrence(w["q"], w["k"], w["v"], w["g"], w["beta"], None, rule="delta",
                                 gate="scalar")
    check_ends("gdn pipelined", T, (o, s), ref)


@pytest.mark.timeout(600)
def test_add_single_pass_max_length():
    import gated_delta_rule_27_amd as la
    T = T_MAX
    x = draw({"q": (1, 1, T, 64), "k": (1, 1, T, 64), "v": (1, 1, T, DV), "g": (1, 1, T)},
             seed=402, unit=("q", "k"))
    o, s = la.chunk_fwd(x["q"], x["k"], x["v"], x["g"], None, None, rule="add", gate="scalar")
    torch.cuda.synchronize()

    def ref(sl):
        w = piece(x, sl)
        return oracle.recurrence(w["q"], w["k"], w["v"], w["g"], None, None, rule="add", gate="scalar")
    check_ends("add single-pass d_k=64", T, (o, s), ref)


@pytest.mark.timeout(600)
def test_kda_two_kernel_max_length():
    import gated_delta_rule_27_amd as la
    T = T_MAX
    x = draw({"q": (1, 1, T, 128), "k": (1, 1, T, 128), "v": (1, 1, T, DV), "g": (1, 1, T, 128),
              "beta": (1, 1, T)}, seed=403, unit=("q", "k"))
    o, s = la.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None, rule="delta", gate="channel")
    torch.cuda.synchronize()

    def ref(sl):
        w = piece(x, sl)
        return oracle.recurrence(w["q"], w["k"], w["v"], w["g"], w["beta"], None, rule="delta",
                                 gate="channel")
    check_ends("kda two-kernel", T, (o, s), ref)


@pytest.mark.timeout(600)
def test_normalized_one_pass_max_length():
    import gated_delta_rule_27_amd as la
    T = T_MAX
    x = draw({"q": (1, 1, T, 128), "k": (1, 1, T, 128), "v": (1, 1, T, DV), "g": (1, 1, T)},
             seed=404, positive=("q", "k"))
    o, s, z = la.chunk_fwd_normalized(x["q"], x["k"], x["v"], x["g"], gate="scalar")
    torch.cuda.synchronize()

    def ref(sl):
        w = piece(x, sl)
        return oracle.normalized(w["q"], w["k"], w["v"], w["g"], None, None, gate="scalar")
    check_ends("normalised one-pass", T, (o, s, z), ref)


@pytest.mark.timeout(600)
def test_deltaproduct_in_place_max_length():
    import gated_delta_rule_27_amd as la
    nh = 2
    T = T_MAX // nh                         # virtual length 2 T = T_MAX - 1
    x = draw({"q": (1, 1, T, 128), "k": (1, 1, T, nh, 128), "v": (1, 1, T, nh, DV), "g": (1, 1, T),
              "beta": (1, 1, T, nh)}, seed=405, unit=("q", "k"))
    o, s = la.deltaproduct_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None, gate="scalar")
    torch.cuda.synchronize()

    def ref(sl):
        w = piece(x, sl)
        return oracle.deltaproduct(w["q"], w["k"], w["v"], w["g"], w["beta"], None, gate="scalar")
    check_ends(f"gated deltaproduct n_h={nh} in place", T, (o, s), ref)


@pytest.mark.timeout(600)
def test_decode_state_past_2g_elements():
    # 8192 sequences x 32 heads x 128 x 128 fp32: 2^32 state elements (16 GiB),
    # so the second half of the heads starts past element 2^31 (byte offsets
    # past 2^33); sampled heads at both ends and on each side of that boundary
    # against the oracle's step
    import gated_delta_rule_27_amd as la
    N, H, d = 8192, 32, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(406)
    state = torch.randn((N, H, d, d), generator=gen, device="cuda") * 0.1
    x = draw({"q": (N, H, d), "k": (N, H, d), "v": (N, H, d), "g": (N, H), "beta": (N, H)},
             seed=407, unit=("q", "k"))
    picks = [(0, 0), (4095, 31), (4096, 0), (8191, 30), (8191, 31)]
    before = [host(state[n, h]) for n, h in picks]
    o = la.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, rule="delta", gate="scalar")
    torch.cuda.synchronize()
    for i, (n, h) in enumerate(picks):
        one = {k2: host(t[n, h])[None, None] for k2, t in x.items()}
        o_ref, s_ref = oracle.decode_step(one["q"], one["k"], one["v"], one["g"], one["beta"],
                                          before[i][None, None], rule="delta", gate="scalar")
        eo = rel_l2(host(o[n, h]), o_ref[0, 0])
        es = rel_l2(host(state[n, h]), s_ref[0, 0])
        note(f"[max] decode head ({n},{h}): rel L2 o {eo:.3e} state {es:.3e}")
        assert eo <= TOL["bf16"] and es <= 1e-5
