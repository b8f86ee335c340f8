"""GPU parity of the full-layer path (the packed input projection GEMM, the
causal conv1d + SiLU, the prefill, the output projection) against the fp64
oracle, each kernel also on its own.

Numbers: the GEMM and conv results are bf16-rounded, so each element must
lie within 0.4 % of the fp64 value (half a bf16 ulp is at most 2^-8 =
0.39 % of the value) plus 1e-4 of the result's rms; the layer output and final state
must meet the prefill's bf16 bar, relative L2 error <= 2e-2, per sequence
(output) and per (sequence, value head) (state).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_linear_04_amd import binding, synth
from tests import gpu_helpers as G
from tests import parity_metrics as PM

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load()
    return torch.device("cuda:0")


def _say(msg):
    print("[case] " + msg, flush=True)


def _bf16(rng, shape, scale=1.0):
    return synth.to_storage(scale * rng.standard_normal(shape), synth.BF16)


def _f64(bits):
    return synth.storage_to_f64(bits, synth.BF16)


def _close_elementwise(y, ref, label):
    y = np.asarray(y, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(y - ref)
    bound = 0.004 * np.abs(ref) + 1e-4 * rms + 1e-30
    worst = float((err / bound).max()) if err.size else 0.0
    print("[parity] %s max err/bound=%.3f max_abs=%.3e rms_ref=%.3e"
          % (label, worst, float(err.max()) if err.size else 0.0, rms), flush=True)
    assert worst <= 1.0, (label, worst)


# shapes reach every tile configuration: 128 x 128 with k-tiles of 32 and
# 64, 128 x 160 (the out_proj shape), 256 x 256 with 32 (K = 96) and 64,
# 256 x 224 (the in_proj shape) and 256 x 192 (4096 x 3072; 2048 x 9000,
# whose last column tile is ragged); the eight-wave kernel (256-row tiles,
# K % 64 = 0) also with a ragged last row tile: 2100 x 12380 (224-wide
# tiles, rows of C not 16-byte multiples, so the per-lane stores) and
# 2100 x 12360 (the 16-byte row stores)
@pytest.mark.parametrize("M,N,K", [(5, 16, 32), (300, 200, 96), (257, 520, 64),
                                   (2048, 2560, 4096), (2048, 12352, 2560),
                                   (4096, 4096, 96), (4096, 4096, 256),
                                   (4096, 3072, 128), (2048, 9000, 512),
                                   (2100, 12380, 256), (2100, 12360, 256)])
def test_gemm_matches_fp64(dev, M, N, K):
    _say("gemm M=%d N=%d K=%d" % (M, N, K))
    rng = np.random.default_rng(7000 + M + N + K)
    A = _bf16(rng, (M, K))
    B = _bf16(rng, (N, K), 0.02)
    C = binding.gemm(G.to_dev(A, dev), G.to_dev(B, dev))
    torch.cuda.synchronize(dev)
    ref = _f64(A) @ _f64(B).T
    _close_elementwise(G.to_f64(C), ref, "gemm %dx%dx%d" % (M, N, K))


def test_gemm_ragged_columns_with_padded_rows(dev):
    # C with a row stride past N (ldc = 208 for N = 203): the 16-byte row
    # stores of the epilogue, a last piece of 3 columns per row, and the
    # padding columns left as they were
    import ctypes
    M, N, K, ldc = 300, 203, 64, 208
    _say("gemm M=%d N=%d K=%d ldc=%d" % (M, N, K, ldc))
    rng = np.random.default_rng(7077)
    A = _bf16(rng, (M, K))
    B = _bf16(rng, (N, K), 0.02)
    Ad, Bd = G.to_dev(A, dev), G.to_dev(B, dev)
    C = torch.full((M, ldc), 7.0, dtype=torch.bfloat16, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    binding._check(binding.load().gdn_gemm_bf16(
        M, N, K, ctypes.c_void_p(Ad.data_ptr()), K, ctypes.c_void_p(Bd.data_ptr()), K,
        ctypes.c_void_p(C.data_ptr()), ldc, ctypes.c_void_p(st)))
    torch.cuda.synchronize(dev)
    Cf = G.to_f64(C)
    _close_elementwise(Cf[:, :N], _f64(A) @ _f64(B).T, "gemm %dx%dx%d ldc=%d" % (M, N, K, ldc))
    assert np.all(Cf[:, N:] == 7.0)


@pytest.mark.parametrize("W", [4, 3])
def test_conv_silu_matches_oracle(dev, W):
    _say("conv W=%d" % W)
    rng = np.random.default_rng(7100 + W)
    T, C = 300, 8192
    x = _bf16(rng, (T, C))
    w = _bf16(rng, (C, W), 0.5)
    y = binding.conv_silu(G.to_dev(x, dev), G.to_dev(w, dev))
    torch.cuda.synchronize(dev)
    ref = oracle.causal_conv_silu(_f64(x), _f64(w))
    _close_elementwise(G.to_f64(y), ref, "conv one sequence W=%d" % W)
    # sequences restart the conv history (an empty one included); the
    # second pattern starts sequences on and just past token-tile edges
    # (multiples of 8) and holds sequences shorter than the window
    for cu in (np.array([0, 5, 5, 130, 300], dtype=np.int32),
               np.array([0, 8, 16, 19, 21, 64, 67, 72, 80, 300], dtype=np.int32)):
        y = binding.conv_silu(G.to_dev(x, dev), G.to_dev(w, dev),
                              cu_seqlens=G.to_dev(cu, dev))
        torch.cuda.synchronize(dev)
        ref = np.concatenate([oracle.causal_conv_silu(_f64(x[s:e]), _f64(w))
                              for s, e in zip(cu[:-1], cu[1:]) if e > s])
        _close_elementwise(G.to_f64(y), ref, "conv varlen W=%d cu=%s" % (W, cu.tolist()))


def _layer_gpu(c, dev, cu=None):
    x = G.to_dev(c["x"], dev)
    W_in_t = G.to_dev(np.ascontiguousarray(c["W_in"].T), dev)
    W_out_t = G.to_dev(np.ascontiguousarray(c["W_out"].T), dev)
    out, S = binding.layer_prefill(
        x, W_in_t, G.to_dev(c["conv_w"], dev), G.to_dev(c["A_log"], dev),
        G.to_dev(c["dt_bias"], dev), G.to_dev(c["norm_w"], dev), W_out_t,
        c["Hk"], c["Hv"], cu_seqlens=None if cu is None else G.to_dev(cu, dev))
    torch.cuda.synchronize(dev)
    return G.to_f64(out), G.to_f64(S)


def _layer_ref(c, s, e):
    return oracle.layer(_f64(c["x"][s:e]), _f64(c["W_in"]), _f64(c["conv_w"]),
                        c["A_log"], c["dt_bias"], c["norm_w"], _f64(c["W_out"]),
                        c["Hk"], c["Hv"])


# Tail budget of the layer's elementwise check (tests/parity_metrics.py):
# the fp64 layer oracle keeps every intermediate unrounded, while the layer
# stores its projections and conv outputs in bf16; the rounding of the gate
# pre-activation a alone moves each decay by up to exp(A_log) |a|
# sigmoid(a + dt_bias) 2^-9 (A_log up to ln 16).  The layer's relative L2
# error is about 6e-3, and out_proj sums 4096 products per element, so the
# per-element error is close to Gaussian with sigma ~ 6e-3 rms: the 2e-2
# bound sits about 3.4 sigma out for elements near zero, where a fraction of
# order 1e-4 lies.  Up to 1e-3 of the elements may exceed their bound; none
# may exceed 4x it (13 sigma), which a wrong element or row always does.
LAYER_TAIL, LAYER_CAP = 1e-3, 4.0


def _check_layer(out, S, refs, bounds, label):
    """Per sequence (layer output) and per (sequence, value head) state:
    relative L2 and every element against the bf16 bar 2e-2
    (tests/parity_metrics.py), with the layer's tail budget."""
    t_o, t_s = PM.Tally(LAYER_TAIL, LAYER_CAP), PM.Tally(LAYER_TAIL, LAYER_CAP)
    for n, ((o_ref, S_ref), (s, e)) in enumerate(zip(refs, bounds)):
        if e == s:
            continue
        t_o.add(out[s:e], o_ref, PM.TOL["bf16"])
        for h in range(S_ref.shape[1]):
            t_s.add(S[n, h], S_ref[0, h], PM.TOL["bf16"])
    print("[parity] %s | out: %r | state: %r" % (label, t_o, t_s), flush=True)
    G.assert_parity(t_o, t_s, label)


@pytest.mark.parametrize("T", [130, 2048])
def test_layer_matches_oracle(dev, T):
    _say("layer T=%d hidden=2560 4B geometry" % T)
    c = synth.layer_case(synth.seed_for(4, T), T=T)
    out, S = _layer_gpu(c, dev)
    _check_layer(out, S, [_layer_ref(c, 0, T)], [(0, T)], "layer T=%d" % T)


def test_layer_hv48(dev):
    # the Hv = 48 variant of the 4B geometry (three value heads per key
    # head) through the whole layer: in_proj 2560 -> 16384 + 96 columns
    _say("layer T=130 hidden=2560 Hk=16 Hv=48")
    c = synth.layer_case(synth.seed_for(4, 48), T=130, Hv=48)
    out, S = _layer_gpu(c, dev)
    _check_layer(out, S, [_layer_ref(c, 0, 130)], [(0, 130)], "layer Hv=48")


def test_layer_varlen(dev):
    _say("layer varlen 70|1|0|100")
    c = synth.layer_case(synth.seed_for(4, 900), T=171)
    cu = np.array([0, 70, 71, 71, 171], dtype=np.int32)
    out, S = _layer_gpu(c, dev, cu)
    bounds = list(zip(cu[:-1], cu[1:]))
    refs = []
    for s, e in bounds:
        if e > s:
            refs.append(_layer_ref(c, s, e))
        else:
            refs.append((None, np.zeros((1, c["Hv"], 128, 128))))
    # an empty sequence keeps the (zero) initial state exactly
    assert np.all(S[2] == 0.0)
    _check_layer(out, S, refs, bounds, "layer varlen")


@pytest.mark.parametrize("W", [4, 2])
def test_conv_history_in_and_out(dev, W):
    # history rows continue each sequence (short and empty ones included);
    # the returned history is each sequence's last W - 1 input rows, exact
    _say("conv with history W=%d, varlen 2|0|1|40|90" % W)
    rng = np.random.default_rng(7200 + W)
    C = 2048
    cu = np.array([0, 2, 2, 3, 43, 133], dtype=np.int32)
    N, T = len(cu) - 1, int(cu[-1])
    x = _bf16(rng, (T, C))
    w = _bf16(rng, (C, W), 0.5)
    hin = _bf16(rng, (N, W - 1, C))
    hin_d = G.to_dev(hin, dev)
    hout_d = torch.full((N, W - 1, C), float("nan"), dtype=torch.bfloat16, device=dev)
    y = binding.conv_silu(G.to_dev(x, dev), G.to_dev(w, dev),
                          cu_seqlens=G.to_dev(cu, dev), hist_in=hin_d, hist_out=hout_d)
    torch.cuda.synchronize(dev)
    ref, href = [], []
    for n, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        if e > s:
            ref.append(oracle.causal_conv_silu(_f64(x[s:e]), _f64(w), _f64(hin[n])))
        href.append(oracle.conv_history(_f64(x[s:e]), W, _f64(hin[n])))
    _close_elementwise(G.to_f64(y), np.concatenate(ref), "conv history W=%d" % W)
    # the history is a copy of input rows: bit-exact
    assert np.array_equal(G.to_f64(hout_d), np.stack(href)), "conv history out"
    # in place (hist_out is hist_in): same rows as above
    y2 = binding.conv_silu(G.to_dev(x, dev), G.to_dev(w, dev),
                           cu_seqlens=G.to_dev(cu, dev), hist_in=hin_d, hist_out=hin_d)
    torch.cuda.synchronize(dev)
    assert torch.equal(y2, y)
    assert torch.equal(hin_d, hout_d)


def test_layer_split_with_carried_states(dev):
    # two layer calls carrying the recurrent state and the conv history match
    # the oracle's one-call result, for a split inside a chunk and inside the
    # first conv window, on two sequences at once
    _say("layer split calls with carried state and conv history")
    c = synth.layer_case(synth.seed_for(4, 901), T=300)
    Hk, Hv = c["Hk"], c["Hv"]
    C = 2 * Hk * 128 + Hv * 128
    lens = [(2, 118), (70, 110)]  # per sequence: tokens in call 1, call 2
    # token layout of the source rows: sequence 0 = rows 0..119, 1 = 120..299
    starts = [0, 120]
    W_in_t = G.to_dev(np.ascontiguousarray(c["W_in"].T), dev)
    W_out_t = G.to_dev(np.ascontiguousarray(c["W_out"].T), dev)
    common = (G.to_dev(c["conv_w"], dev), G.to_dev(c["A_log"], dev),
              G.to_dev(c["dt_bias"], dev), G.to_dev(c["norm_w"], dev), W_out_t, Hk, Hv)
    hist = torch.zeros((2, 3, C), dtype=torch.bfloat16, device=dev)
    S = None
    outs = [[], []]
    for call in range(2):
        rows = [np.arange(starts[n] + (0 if call == 0 else lens[n][0]),
                          starts[n] + lens[n][0] + (0 if call == 0 else lens[n][1]))
                for n in range(2)]
        xs = np.concatenate([c["x"][r] for r in rows])
        cu = np.array([0, len(rows[0]), len(rows[0]) + len(rows[1])], dtype=np.int32)
        out, S = binding.layer_prefill(
            G.to_dev(xs, dev), W_in_t, *common, state_in=S,
            cu_seqlens=G.to_dev(cu, dev), conv_state_in=hist, conv_state_out=hist)
        torch.cuda.synchronize(dev)
        o = G.to_f64(out)
        outs[0].append(o[:cu[1]])
        outs[1].append(o[cu[1]:])
    S = G.to_f64(S)
    t_o, t_s = PM.Tally(LAYER_TAIL, LAYER_CAP), PM.Tally(LAYER_TAIL, LAYER_CAP)
    for n in range(2):
        s0, tot = starts[n], sum(lens[n])
        o_ref, S_ref = _layer_ref(c, s0, s0 + tot)
        t_o.add(np.concatenate(outs[n]), o_ref, PM.TOL["bf16"])
        for h in range(Hv):
            t_s.add(S[n, h], S_ref[0, h], PM.TOL["bf16"])
    print("[parity] layer split carried | out: %r | state: %r" % (t_o, t_s), flush=True)
    G.assert_parity(t_o, t_s, "layer split carried")


def layer_sweep_case(i: int):
    """Seeded layer batch i: hidden 256..1024, 4..32 value heads over 1..16
    key heads (counts whose in_proj column segments start off the 8- and
    16-column grid among them, e.g. b | a at 12 value heads), conv width
    2..4, 1..4 sequences whose lengths mix 0, 1, 63..65 with uniform
    lengths up to 200."""
    rng = np.random.default_rng(97_000 + i)
    hidden = int(rng.choice([256, 768, 1024]))
    Hv = int(rng.choice([4, 6, 8, 12, 16, 24, 32]))
    Hk = int(rng.choice([h for h in (1, 2, 3, 4, 8, 16) if Hv % h == 0]))
    W = int(rng.integers(2, 5))
    N = int(rng.integers(1, 5))
    lens = [int(rng.choice([0, 1, 63, 64, 65])) if rng.random() < 0.4 else int(rng.integers(1, 201))
            for _ in range(N)]
    if sum(lens) == 0:
        lens[-1] = 70
    c = synth.layer_case(98_000 + i, T=sum(lens), hidden=hidden, Hk=Hk, Hv=Hv,
                         conv_width=W)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    return c, cu


@pytest.mark.parametrize("i", range(8))
def test_layer_sweep(dev, i):
    c, cu = layer_sweep_case(i)
    _say("layer sweep %d hidden=%d Hk=%d Hv=%d W=%d lens=%s" % (
        i, c["hidden"], c["Hk"], c["Hv"], c["conv_w"].shape[1], np.diff(cu).tolist()))
    out, S = _layer_gpu(c, dev, cu)
    bounds = list(zip(cu[:-1], cu[1:]))
    refs = []
    for n, (s, e) in enumerate(bounds):
        if e == s:
            # an empty sequence keeps its (zero) initial state exactly
            assert np.all(S[n] == 0.0), n
            refs.append((None, None))
            continue
        refs.append(oracle.layer(_f64(c["x"][s:e]), _f64(c["W_in"]), _f64(c["conv_w"]),
                                 c["A_log"], c["dt_bias"], c["norm_w"], _f64(c["W_out"]),
                                 c["Hk"], c["Hv"]))
    _check_layer(out, S, refs, bounds, "layer sweep%d" % i)


def test_layer_graph_replay_matches_eager(dev):
    # the whole layer (GEMM, conv with history in and out, prefill, GEMM)
    # captured once and replayed three times, each replay bitwise equal to
    # the eager call, with eager work and synchronisation between replays
    _say("layer graph capture/replay T=200 hidden=512 varlen 120|80")
    c = synth.layer_case(synth.seed_for(4, 950), T=200, hidden=512)
    cu = G.to_dev(np.array([0, 120, 200], dtype=np.int32), dev)
    x = G.to_dev(c["x"], dev)
    W_in_t = G.to_dev(np.ascontiguousarray(c["W_in"].T), dev)
    W_out_t = G.to_dev(np.ascontiguousarray(c["W_out"].T), dev)
    conv_w = G.to_dev(c["conv_w"], dev)
    A_log, dt_bias, norm_w = (G.to_dev(c[k], dev) for k in ("A_log", "dt_bias", "norm_w"))
    C, W = c["conv_w"].shape
    rng = np.random.default_rng(951)
    hist_in = G.to_dev(synth.to_storage(rng.standard_normal((2, W - 1, C)), synth.BF16), dev)
    S_in = torch.from_numpy((0.02 * rng.standard_normal((2, c["Hv"], 128, 128))).astype(
        np.float32)).to(dev)
    desc = binding.make_layer_desc(2, 200, 512, c["Hk"], c["Hv"], W)
    ws = torch.empty(binding.layer_workspace_size(desc), dtype=torch.uint8, device=dev)
    out = torch.empty(200, 512, dtype=torch.bfloat16, device=dev)
    S_out = torch.empty_like(S_in)
    hist_out = torch.empty_like(hist_in)

    def call():
        binding.layer_prefill(x, W_in_t, conv_w, A_log, dt_bias, norm_w, W_out_t, c["Hk"],
                              c["Hv"], state_in=S_in, cu_seqlens=cu, conv_state_in=hist_in,
                              conv_state_out=hist_out, out=out, state_out=S_out, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = (out.clone(), S_out.clone(), hist_out.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        out.fill_(float("nan"))
        S_out.fill_(float("nan"))
        hist_out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]), rep
        assert torch.equal(S_out, ref[1]), rep
        assert torch.equal(hist_out, ref[2]), rep


def test_layer_fused_conv_matches_separate_conv(dev):
    # the conv applied inside the prefill's first kernel gives the layer the
    # bits of the conv as a kernel of its own: outputs, states and the conv
    # history carried out (in place), on a varlen batch with history in
    _say("layer fused vs separate conv, varlen 70|1|0|100 with conv history")
    c = synth.layer_case(synth.seed_for(4, 901), T=171)
    cu = G.to_dev(np.array([0, 70, 71, 71, 171], dtype=np.int32), dev)
    rng = np.random.default_rng(901)
    hist = _bf16(rng, (4, 3, c["conv_ch"]))
    x = G.to_dev(c["x"], dev)
    W_in_t = G.to_dev(np.ascontiguousarray(c["W_in"].T), dev)
    W_out_t = G.to_dev(np.ascontiguousarray(c["W_out"].T), dev)
    common = (G.to_dev(c["conv_w"], dev), G.to_dev(c["A_log"], dev), G.to_dev(c["dt_bias"], dev),
              G.to_dev(c["norm_w"], dev), W_out_t, c["Hk"], c["Hv"])
    S0 = torch.randn(4, c["Hv"], 128, 128, device=dev) * 0.02
    res = []
    for fused in (1, 0):
        h = G.to_dev(hist, dev)
        out, S = binding.layer_prefill(x, W_in_t, *common, state_in=S0, cu_seqlens=cu,
                                       conv_state_in=h, conv_state_out=h, conv_fused=fused)
        torch.cuda.synchronize(dev)
        res.append((out, S, h))
    assert torch.equal(res[0][0], res[1][0])
    assert torch.equal(res[0][1], res[1][1])
    assert torch.equal(res[0][2], res[1][2])
