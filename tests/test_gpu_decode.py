"""GPU parity of the codec and the decode step against the CPU oracle,
through the C ABI (ops -> ctypes -> libgdnq.so)."""

import numpy as np
import pytest
import torch

import oracle as O
import oracle_pool
import workloads as wl
from conftest import read_golden
from gpu_util import (DEV, assert_free_scales, OUT_TOL_BF16, OUT_TOL_F32, Guarded, assert_codes, assert_scales,
                      dev, host, max_rel_err)

pytestmark = pytest.mark.gpu

if DEV is not None:
    from quantized_recurrent_state_gdnq_amd import ops


# ---------------------------------------------------------------- codec
@pytest.mark.parametrize("d", [64, 128])
def test_codec_golden_rows_bitwise(d):
    g = read_golden("codec_rows.txt")
    rows = []
    for row in g["row"]:
        x = np.zeros(d, np.float32)
        vals = [float(v) for v in row.split()]
        x[:len(vals)] = vals
        rows.append(x)
    S = np.stack(rows)
    codes, scales = ops.quantize_state(dev(S))
    torch.cuda.synchronize()
    for i, (sc, cd) in enumerate(zip(g["scale"], g["codes"])):
        exp = [int(v) for v in cd.split()]
        assert host(codes)[i, :len(exp)].tolist() == exp
        assert np.all(host(codes)[i, len(exp):] == 0)
        assert host(scales)[i] == np.float32(float(sc))


@pytest.mark.parametrize("state_bits", [8, 4])
def test_codec_subnormal_scale(state_bits):
    """The golden row whose scale is a subnormal (2^-140 for 8 bits): the
    library's codec divides, so the codes are the exact quotients.  The
    4-bit codec is checked against the oracle's qmax = 7 on the same row."""
    g = read_golden("codec_subnormal.txt")
    f = 2.0 ** int(g["pow2"][0])
    x = np.zeros((1, 128), np.float32)
    vals = [float(v) for v in g["row"][0].split()]
    x[0, :len(vals)] = np.array(vals) * f
    codes, scales = ops.quantize_state(dev(x), state_bits=state_bits)
    torch.cuda.synchronize()
    rc, rs = O.quantize_rows(x, qmax=127 if state_bits == 8 else 7)
    got = host(codes)
    if state_bits == 4:
        u = got.view(np.uint8).astype(np.int16)
        lo, hi = u & 0xF, u >> 4
        got = np.stack([np.where(lo > 7, lo - 16, lo), np.where(hi > 7, hi - 16, hi)], -1).reshape(1, 128)
    assert got.tolist() == rc.tolist()
    assert host(scales)[0] == rs[0]
    if state_bits == 8:
        assert got[0, :len(vals)].tolist() == [int(v) for v in g["codes"][0].split()]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rows", [1, 17, 4099])
@pytest.mark.parametrize("wht", [False, True])
def test_codec_random(d, rows, wht):
    g = np.random.default_rng(rows + d)
    S = (g.standard_normal((rows, d)) * np.exp(g.uniform(-4, 4, (rows, 1)))).astype(np.float32)
    S[rows // 2] = 0.0
    if rows > 100:
        S[3, 5] = 40.0  # an outlier channel
    St = Guarded((rows, d), torch.float32).set(S)
    C = Guarded((rows, d), torch.int8)
    Sc = Guarded((rows,), torch.float32)
    ops.quantize_state(St.t, C.t, Sc.t, wht=wht)
    torch.cuda.synchronize()
    assert C.guards_intact() and Sc.guards_intact()
    ref_in = O.gdnq_oracle.rotate(S, np.float32) if wht else S
    rc, rs = O.quantize_rows(ref_in)
    if wht:
        assert_codes(host(C.t), rc, "codec+wht")
        assert_scales(host(Sc.t), rs, "codec+wht")
    else:
        assert np.array_equal(host(C.t), rc)
        assert np.array_equal(host(Sc.t), rs)


# ---------------------------------------------------------------- decode
def _run_decode(d, W, in_dt, out_dt, wht=False):
    """One GPU decode step on generator output `d`; returns host results and
    the quantized initial state (the oracle's codec quantizes it)."""
    B, H, dv, dk = d["state"].shape
    codes, scales = O.quantize_rows(O.gdnq_oracle.rotate(d["state"], np.float32) if wht
                                    else d["state"])
    g = {
        "codes": Guarded((B, H, dv, dk), torch.int8).set(codes),
        "scales": Guarded((B, H, dv), torch.float32).set(scales),
        "buf_k": Guarded((B, H, W, dk), torch.float32).set(d["buf_k"]),
        "buf_v": Guarded((B, H, W, dv), torch.float32).set(d["buf_v"]),
        "buf_alpha": Guarded((B, H, W), torch.float32).set(d["buf_alpha"]),
        "buf_beta": Guarded((B, H, W), torch.float32).set(d["buf_beta"]),
        "fill_out": Guarded((B,), torch.int32),
        "o": Guarded((B, H, dv), out_dt),
    }
    fin = dev(d["fill"])
    ops.decode_step(dev(d["q"], in_dt), dev(d["k"], in_dt), dev(d["v"], in_dt), dev(d["alpha"]),
                    dev(d["beta"]), g["codes"].t, g["scales"].t, g["buf_k"].t, g["buf_v"].t,
                    g["buf_alpha"].t, g["buf_beta"].t, fin, g["fill_out"].t, g["o"].t, wht=wht)
    torch.cuda.synchronize()
    for name, x in g.items():
        assert x.guards_intact(), f"write outside {name}"
    assert np.array_equal(host(fin), d["fill"]), "fill_in was modified"
    return {k: host(v.t) for k, v in g.items()}, codes, scales


def _check_decode(d, W, got, codes, scales, tol, wht=False):
    ref = O.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], codes, scales, d["buf_k"],
                        d["buf_v"], d["buf_alpha"], d["buf_beta"], d["fill"], W, rot=wht)
    o, rc, rs, rbk, rbv, rba, rbb, rfill = ref
    err = max_rel_err(got["o"], o)
    assert err <= tol, f"o max relative error {err:.3e} > {tol}"
    assert np.array_equal(got["fill_out"], rfill)
    closing = d["fill"] + 1 == W
    # untouched sequences: state bitwise unchanged, appended slot exact
    assert np.array_equal(got["codes"][~closing], codes[~closing])
    assert np.array_equal(got["scales"][~closing], scales[~closing])
    for bi in np.nonzero(~closing)[0]:
        f = d["fill"][bi]
        if wht:
            np.testing.assert_allclose(got["buf_k"][bi, :, f], rbk[bi, :, f], rtol=0, atol=2e-6)
        else:
            assert np.array_equal(got["buf_k"][bi, :, f], rbk[bi, :, f])
        assert np.array_equal(got["buf_v"][bi, :, f], rbv[bi, :, f])
        assert np.array_equal(got["buf_alpha"][bi, :, f], rba[bi, :, f])
        assert np.array_equal(got["buf_beta"][bi, :, f], rbb[bi, :, f])
        # slots below the fill are not touched
        assert np.array_equal(got["buf_k"][bi, :, :f], d["buf_k"][bi, :, :f])
    if closing.any():
        assert_codes(got["codes"][closing], rc[closing], "closing codes")
        assert_scales(got["scales"][closing], rs[closing], "closing scales")
    return err


DECODE_CASES = [
    # (B, H, dk, dv, W, in_dtype, out_dtype, wht, forced fills)
    (4, 3, 128, 128, 8, torch.bfloat16, torch.bfloat16, False, [0, 3, 7, 7]),
    (4, 3, 128, 128, 8, torch.bfloat16, torch.float32, True, [7, 1, 6, 0]),
    (3, 2, 128, 64, 5, torch.bfloat16, torch.bfloat16, False, [4, 2, 0]),
    (3, 2, 64, 128, 5, torch.float32, torch.float32, False, [4, 2, 0]),
    (2, 5, 64, 64, 16, torch.float32, torch.float32, True, [15, 9]),
    (3, 2, 128, 128, 1, torch.bfloat16, torch.bfloat16, False, [0, 0, 0]),
    (2, 2, 128, 128, 64, torch.bfloat16, torch.bfloat16, False, [63, 62]),
    (3, 2, 64, 64, 8, torch.bfloat16, torch.float32, False, [7, 3, 0]),
    (3, 2, 64, 128, 8, torch.bfloat16, torch.bfloat16, True, [2, 7, 5]),
    (2, 3, 128, 64, 64, torch.bfloat16, torch.float32, True, [63, 40]),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"B{c[0]}H{c[1]}dk{c[2]}dv{c[3]}W{c[4]}wht{int(c[7])}")
def test_decode_step_cases(case):
    B, H, dk, dv, W, in_dt, out_dt, wht, fills = case
    d = wl.decode_batch(B=B, H=H, dk=dk, dv=dv, W=W, seed=B * 7 + W, fill=np.array(fills))
    if in_dt == torch.float32:  # fp32 inputs need not be bf16-representable
        g = np.random.default_rng(W)
        d["q"] = wl.l2norm(g.standard_normal(d["q"].shape).astype(np.float32))
        d["k"] = wl.l2norm(g.standard_normal(d["k"].shape).astype(np.float32))
        d["v"] = g.standard_normal(d["v"].shape).astype(np.float32)
    got, codes, scales = _run_decode(d, W, in_dt, out_dt, wht)
    tol = OUT_TOL_F32 if (in_dt == torch.float32 and out_dt == torch.float32) else OUT_TOL_BF16
    _check_decode(d, W, got, codes, scales, tol, wht)


def test_decode_batch64_heads32_window64():
    """The one-step decode workload at its full size: B=64, H=32, d=128,
    W=64, drawn fills in 0..63 (sequences at fill 63 close their window)."""
    fill = wl.decode_batch(B=64, H=32, dk=128, dv=128, W=64, seed=0)["fill"]
    fill[:2] = 63  # make sure at least two sequences close
    d = wl.decode_batch(B=64, H=32, dk=128, dv=128, W=64, seed=0, fill=fill)
    got, codes, scales = _run_decode(d, 64, torch.bfloat16, torch.bfloat16)
    err = _check_decode(d, 64, got, codes, scales, OUT_TOL_BF16)
    print(f"B64 H32 decode: max rel err {err:.3e}")


def test_decode_max_batch():
    """The largest batch a call takes, B=1024 (H=2, d=64, W=64): the fill
    scan runs over 16 blocks of 64 sequences, the open sequences are sorted
    by fill across all of them, and closing sequences sit in the first, a
    middle and the last block."""
    B, H, d, W = 1024, 2, 64, 64
    fill = wl.decode_batch(B=B, H=H, dk=d, dv=d, W=W, seed=11)["fill"]
    fill[[0, 63, 64, 511, 1000, 1023]] = W - 1
    d_ = wl.decode_batch(B=B, H=H, dk=d, dv=d, W=W, seed=11, fill=fill)
    got, codes, scales = _run_decode(d_, W, torch.bfloat16, torch.bfloat16)
    err = _check_decode(d_, W, got, codes, scales, OUT_TOL_BF16)
    print(f"B1024 H2 d64 decode: max rel err {err:.3e}, {int((fill == W - 1).sum())} closing")


@pytest.mark.parametrize("wht", [False, True])
def test_decode_strong_decay_full_window(wht):
    """Fast-forgetting heads: decays drawn from U(0.02, 0.2), so the product
    of a full window's 64 decays (~1e-64) is far below fp32's range.  Closing
    and open sequences must stay finite and match the oracle."""
    W = 64
    d = wl.decode_batch(B=4, H=2, dk=128, dv=128, W=W, seed=77, fill=np.array([63, 63, 40, 10]))
    g = np.random.default_rng(78)
    live = ~np.isnan(d["buf_alpha"])
    d["buf_alpha"] = np.where(live, g.uniform(0.02, 0.2, live.shape), np.nan).astype(np.float32)
    d["alpha"] = g.uniform(0.02, 0.2, d["alpha"].shape).astype(np.float32)
    got, codes, scales = _run_decode(d, W, torch.bfloat16, torch.float32, wht)
    assert np.isfinite(got["o"]).all() and np.isfinite(got["scales"]).all()
    _check_decode(d, W, got, codes, scales, OUT_TOL_BF16, wht)


def test_decode_single_head_fp32_256_steps():
    """Single head, d=64, W=16, fp32 inputs, 256 decode steps from a zero
    state: every output within 1e-3 of the oracle, final state within the
    code bar after 16 requantizations."""
    T, d, W = 256, 64, 16
    x = wl.single_head_fp32(T=T, d=d, seed=0)
    ref = O.run_windowed(x["q"][:, None], x["k"][:, None], x["v"][:, None], x["alpha"][:, None],
                         x["beta"][:, None], W=W)
    st = ops.DecodeState(torch.zeros((1, 1, d, d), dtype=torch.int8, device=DEV),
                         torch.zeros((1, 1, d), dtype=torch.float32, device=DEV), W)
    outs = []
    for t in range(T):
        o = st.step(dev(x["q"][t][None, None]), dev(x["k"][t][None, None]),
                    dev(x["v"][t][None, None]), dev(x["alpha"][t:t + 1][None]),
                    dev(x["beta"][t:t + 1][None]))
        outs.append(o)
    torch.cuda.synchronize()
    got = np.stack([host(o)[0, 0] for o in outs])
    err = max_rel_err(got, ref["o"][:, 0])
    assert err <= OUT_TOL_F32, err
    assert_codes(host(st.codes)[0, 0], ref["codes"][0], "final codes")
    assert_scales(host(st.scales)[0, 0], ref["scale"][0], "final scales")
    assert int(host(st.fill)[0]) == 0


@pytest.mark.parametrize("wht", [False, True])
def test_decode_multi_window(wht):
    """40 consecutive decode steps (5 windows of 8) on a small batch carrying
    codes, scales, buffer and fills, staggered fills so windows close at
    different steps.

    Teacher-forced: every step, the oracle starts from the GPU's state before
    the step, so each requantization is compared on identical inputs (codes
    +-1 on <= 0.1%, scales 1e-5).  Free-running: the oracle also runs on its
    own; outputs stay within 2e-2 and codes within +-1 on <= 0.1%.  A +-1
    flip at one window close is a one-code-unit change of one entry; the
    transitions are non-expansive, so the row's next absmax moves by at most
    one old code unit: about 1/127 relative.  Free-running scales are held
    to 2/127 (two compounded flips)."""
    B, H, dk, dv, W, T = 3, 2, 128, 128, 8, 40
    d0 = wl.decode_batch(B=B, H=H, dk=dk, dv=dv, W=W, seed=5, fill=np.array([0, 3, 7]))
    S0 = O.gdnq_oracle.rotate(d0["state"], np.float32) if wht else d0["state"]
    codes, scales = O.quantize_rows(S0)
    st = ops.DecodeState(dev(codes), dev(scales), W, fill=dev(d0["fill"]), wht=wht)
    st.buf_k.copy_(dev(d0["buf_k"]))
    st.buf_v.copy_(dev(d0["buf_v"]))
    st.buf_alpha.copy_(dev(d0["buf_alpha"]))
    st.buf_beta.copy_(dev(d0["buf_beta"]))
    fr = [codes, scales, d0["buf_k"], d0["buf_v"], d0["buf_alpha"], d0["buf_beta"], d0["fill"]]
    worst_tf = worst_fr = 0.0
    for t in range(T):
        x = wl.decode_tokens(B=B, H=H, dk=dk, dv=dv, step=t, seed=11)
        before = [host(z).copy() for z in (st.codes, st.scales, st.buf_k, st.buf_v, st.buf_alpha,
                                           st.buf_beta, st.fill)]
        o = st.step(dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16),
                    dev(x["v"], torch.bfloat16), dev(x["alpha"]), dev(x["beta"]),
                    out_dtype=torch.float32)
        go = host(o)
        # teacher-forced
        ro, rc, rs, _, _, _, _, rfill = O.decode_step(x["q"], x["k"], x["v"], x["alpha"],
                                                      x["beta"], *before, W, rot=wht)
        worst_tf = max(worst_tf, max_rel_err(go, ro))
        assert np.array_equal(host(st.fill), rfill)
        closing = before[6] + 1 == W
        assert np.array_equal(host(st.codes)[~closing], before[0][~closing])
        if closing.any():
            assert_codes(host(st.codes)[closing], rc[closing], f"step {t} codes")
            assert_scales(host(st.scales)[closing], rs[closing], f"step {t} scales")
        # free-running
        fo, *fr = O.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *fr, W, rot=wht)
        worst_fr = max(worst_fr, max_rel_err(go, fo))
    assert worst_tf <= OUT_TOL_BF16, worst_tf
    assert worst_fr <= OUT_TOL_BF16, worst_fr
    assert_codes(host(st.codes), fr[0], "free-running codes after 5 windows")
    assert_free_scales(host(st.scales), fr[1], f"decode 5 windows wht={wht}")


@pytest.mark.parametrize("grid,open_waves", [(0, 0), (768, 1024), (3, 1), (5, 6), (2, 1000), (40, 7)])
def test_decode_schedules(grid, open_waves):
    """The same mixed open/closing batch under different persistent grids and
    open-wave counts (gdnq_decode_set_schedule): one wave running every open
    head in turn, a single close workgroup looping over all close jobs, and
    the default.  d_k = d_v = 128, W = 16."""
    from quantized_recurrent_state_gdnq_amd import _lib
    _lib.check(_lib.decode_set_schedule(grid, open_waves))
    try:
        d = wl.decode_batch(B=6, H=4, dk=128, dv=128, W=16, seed=grid + open_waves,
                            fill=np.array([15, 0, 7, 15, 14, 3]))
        got, codes, scales = _run_decode(d, 16, torch.bfloat16, torch.float32)
    finally:
        _lib.check(_lib.decode_set_schedule(0, 0))
    _check_decode(d, 16, got, codes, scales, OUT_TOL_BF16)


@pytest.mark.parametrize("H,fill", [(5, [2, 15]), (3, [9, 15, 0]), (1, [4])])
def test_decode_odd_open_heads(H, fill):
    """Odd numbers of heads and open heads (H=5 with one closing sequence: 5
    open heads; H=3: 6; H=1, one sequence: 1).  W = 16, d = 128, bf16
    inputs."""
    d = wl.decode_batch(B=len(fill), H=H, dk=128, dv=128, W=16, seed=40 + H, fill=np.array(fill))
    got, codes, scales = _run_decode(d, 16, torch.bfloat16, torch.float32)
    _check_decode(d, 16, got, codes, scales, OUT_TOL_BF16)


def test_decode_batch256_1024_steps():
    """The large-batch decode workload at its full size: B=256, H=32,
    d=128, W=64, fills drawn U{0..63}, 1024 consecutive steps, so every
    sequence closes 16 windows.  Per-step tokens cycle through 13 drawn sets
    (13 is prime to W).

    * Gate: every window close of 17 sampled sequences, all 32 heads each
      (272 closes of 32 heads), is compared with the oracle started from the
      GPU's own state before the step (teacher-forced): codes +-1 on
      <= 0.1%, scales within 1e-5.
    * Three of those sequences x two heads are also followed by the oracle on
      its own: outputs within 2e-2 at every step."""
    B, H, d, W, T, NP = 256, 32, 128, 64, 1024, 13
    d0 = wl.decode_batch(B=B, H=H, dk=d, dv=d, W=W, seed=3)
    codes, scales = O.quantize_rows(d0["state"])
    ib, ih = np.array([0, 101, 255]), np.array([0, 31])
    tf = np.unique(np.r_[np.arange(0, B, 17), ib])  # sequences whose every close is checked

    def sub(a):
        return np.ascontiguousarray(a[ib][:, ih])

    st = ops.DecodeState(dev(codes), dev(scales), W, fill=dev(d0["fill"]))
    for name in ("buf_k", "buf_v", "buf_alpha", "buf_beta"):
        getattr(st, name).copy_(dev(d0[name]))
    fr = [sub(codes), sub(scales), sub(d0["buf_k"]), sub(d0["buf_v"]), sub(d0["buf_alpha"]),
          sub(d0["buf_beta"]), d0["fill"][ib].copy()]
    del d0, codes, scales
    pool = [wl.decode_tokens(B=B, H=H, dk=d, dv=d, step=i, seed=9) for i in range(NP)]
    tok = [[dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16), dev(x["v"], torch.bfloat16),
            dev(x["alpha"]), dev(x["beta"])] for x in pool]
    tib, tih = torch.from_numpy(ib).to(DEV), torch.from_numpy(ih).to(DEV)

    got = torch.empty((T, len(ib), len(ih), d), dtype=torch.float32, device=DEV)
    fill_all = host(st.fill).astype(np.int64)
    ref_o = np.empty((T, len(ib), len(ih), d), np.float32)
    closes = []
    with oracle_pool.pool() as ex:
        for t in range(T):
            cs = tf[fill_all[tf] + 1 == W]  # checked sequences closing at this step
            if len(cs):
                ts = torch.from_numpy(cs).to(DEV)
                before = [host(z.index_select(0, ts)) for z in (st.codes, st.scales, st.buf_k, st.buf_v,
                                                                 st.buf_alpha, st.buf_beta)]
                before.append(fill_all[cs].copy())
            o = st.step(*tok[t % NP], out_dtype=torch.float32)
            got[t] = o.index_select(0, tib).index_select(1, tih)
            x = pool[t % NP]
            if len(cs):
                xc = [np.ascontiguousarray(x[n][cs]) for n in ("q", "k", "v", "alpha", "beta")]
                fut = oracle_pool.submit(ex, "decode_close", xc, before, W)
                closes.append((t, fut, host(st.codes.index_select(0, ts)), host(st.scales.index_select(0, ts))))
            xs = [sub(x[n]) for n in ("q", "k", "v", "alpha", "beta")]
            ref_o[t], *fr = O.decode_step(*xs, *fr, W)
            fill_all = np.where(fill_all + 1 == W, 0, fill_all + 1)
        torch.cuda.synchronize()
        n_close = 0
        for t, fut, gc, gs in closes:
            rc, rs = fut.result()
            assert_codes(gc, rc, f"step {t} codes")
            assert_scales(gs, rs, f"step {t} scales")
            n_close += len(gc)
    g = host(got)
    worst_fr = 0.0
    for t in range(T):
        worst_fr = max(worst_fr, max_rel_err(g[t], ref_o[t]))
    assert n_close == len(tf) * 16
    assert np.array_equal(host(st.fill), fill_all)
    assert worst_fr <= OUT_TOL_BF16, worst_fr
    print(f"B256 H32 1024 steps: {n_close} sequence closes x 32 heads teacher-forced, "
          f"free-running max rel err {worst_fr:.3e}")


def test_decode_bound_launcher_matches_step():
    """DecodeState.bind (validated once, prebuilt arguments) runs the same
    steps as DecodeState.step: 20 steps over three windows of 8, bitwise."""
    B, H, d, W = 3, 2, 128, 8
    d0 = wl.decode_batch(B=B, H=H, dk=d, dv=d, W=W, seed=21, fill=np.array([0, 5, 7]))
    codes, scales = O.quantize_rows(d0["state"])
    sts = []
    for _ in range(2):
        st = ops.DecodeState(dev(codes), dev(scales), W, fill=dev(d0["fill"]))
        for name in ("buf_k", "buf_v", "buf_alpha", "buf_beta"):
            getattr(st, name).copy_(dev(d0[name]))
        sts.append(st)
    tok = [torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    ab = [torch.empty((B, H), dtype=torch.float32, device=DEV) for _ in range(2)]
    o_b = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
    launch = sts[1].bind(*tok, *ab, o=o_b)
    for t in range(20):
        x = wl.decode_tokens(B=B, H=H, dk=d, dv=d, step=t, seed=22)
        for dst, name in zip(tok, ("q", "k", "v")):
            dst.copy_(dev(x[name], torch.bfloat16))
        for dst, name in zip(ab, ("alpha", "beta")):
            dst.copy_(dev(x[name]))
        o_s = sts[0].step(*tok, *ab)
        launch()
        torch.cuda.synchronize()
        assert torch.equal(o_s, o_b), f"step {t}"
    for name in ("codes", "scales", "fill"):
        assert torch.equal(getattr(sts[0], name), getattr(sts[1], name)), name
    for name in ("buf_k", "buf_v"):  # slots never written keep their NaN poison
        assert torch.allclose(getattr(sts[0], name), getattr(sts[1], name), rtol=0, atol=0,
                              equal_nan=True), name
