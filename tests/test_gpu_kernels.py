"""Kernel-level parity of the HIP path against the CPU oracle (GPU only).

Integer, byte and index work is compared bit for bit; fp64 tables within a
few ulps.  Every call goes through the C ABI (libark.so) via the binding.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
from speech_decoder_int8_amd import ark  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(x):
    torch.cuda.synchronize()
    return x.cpu().numpy()


@pytest.mark.parametrize("n,k", [(37, 64), (300, 2048), (129, 11008)])
def test_prep_weight_bit_exact(n, k):
    rng = np.random.default_rng(n * 31 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[3] = 0.0                                   # a zero row
    w[5, 7] = 0.5                                # a dominant element
    codes, scale, colsum = ark.prep_weight(t(w))
    qo, so = oracle.prep_weight(w)
    assert np.array_equal(host(codes), qo)
    assert np.array_equal(host(scale), so)
    assert np.array_equal(host(colsum), qo.astype(np.int64).sum(1).astype(np.int32))


def test_rope_table_matches_oracle():
    for T, theta in ((512, 1e6), (1024, 1e6), (64, 1e4)):
        c, s = ark.rope_table(T, 128, theta)
        co, so = oracle.rope_tables(T, 128, theta)
        assert np.allclose(host(c), co, rtol=0, atol=4e-16 * np.maximum(1, np.arange(T))[:, None])
        assert np.allclose(host(s), so, rtol=0, atol=4e-16 * np.maximum(1, np.arange(T))[:, None])


# row kernels: rows held in registers (K <= 2048) or a workgroup per row;
# quantisation a workgroup per row (few rows) or a wave per row (>= 1024
# rows); K % 4 != 0 takes the scalar forms
@pytest.mark.parametrize("B,R,K", [(1, 1, 2048), (3, 7, 2048), (2, 49, 11008), (1, 5, 300),
                                   (2, 3, 301), (2, 600, 256), (3, 400, 3001)])
def test_dynquant_bit_exact(B, R, K):
    rng = np.random.default_rng(B * 100 + R)
    x = (rng.standard_normal((B, R, K)) * rng.uniform(0.1, 5, (B, 1, 1))).astype(np.float32)
    if B > 1:
        x[1] = np.abs(x[1])                      # a tensor with no negative value
    x[0, 0, :3] = 0.0
    codes, scale, zp = ark.test_dynquant(t(x))
    codes, scale, zp = host(codes), host(scale), host(zp)
    for b in range(B):
        qo, so, zo = oracle.dynquant(x[b])
        assert np.array_equal(codes[b], qo) and scale[b] == so and zp[b] == int(zo)


def test_dynquant_all_zero_tensor():
    x = np.zeros((1, 2, 256), np.float32)
    codes, scale, zp = ark.test_dynquant(t(x))
    assert not host(codes).any() and host(scale)[0] == 0 and host(zp)[0] == 0


# use_gemm: 0 decode GEMV, 1 the GEMM as the decoder dispatches it, 2 the tiled GEMM
@pytest.mark.parametrize("use_gemm", [0, 1, 2])
@pytest.mark.parametrize("B,R,n,k", [(1, 1, 300, 2048), (2, 2, 2560, 2048), (1, 3, 96, 11008),
                                     (3, 67, 333, 2048), (2, 16, 130, 1024),
                                     # M <= 32: the few-row kernel (K split, ragged rows, one step)
                                     (32, 1, 700, 2048), (4, 8, 256, 128), (1, 31, 4100, 256),
                                     (16, 1, 2048, 11008),
                                     # 32 < M < 128: the few-row kernel once per 32 rows
                                     (1, 49, 700, 2048), (3, 41, 300, 1024),
                                     # M >= 128: the large-tile prefill GEMM (ragged and whole tiles,
                                     # several tiles per CU, K of 3 steps)
                                     (2, 100, 2560, 2048), (1, 256, 512, 1024), (1, 130, 200, 11008),
                                     (3, 101, 700, 2048), (1, 600, 513, 1024), (3, 400, 8000, 256),
                                     (1, 200, 300, 192),
                                     # few tiles: K split over workgroups (128- and 256-row tiles)
                                     (2, 600, 513, 1024), (1, 1030, 256, 2048)])
def test_qlinear_bit_exact(use_gemm, B, R, n, k):
    if use_gemm == 0 and B * R > 4:
        pytest.skip("the decode GEMV takes at most 4 rows")
    rng = np.random.default_rng(n + k + B * R)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    bias = (rng.standard_normal(n) * 0.02).astype(np.float32)
    codes = rng.integers(0, 256, (B, R, k)).astype(np.uint8)
    codes[0, 0, :] = 255                           # extreme accumulators
    scale = rng.uniform(0.001, 0.05, B).astype(np.float32)
    zp = rng.integers(0, 256, B).astype(np.uint8)
    zp[0] = 0
    W = ark.QLinear.from_f32(t(w), t(bias))
    acc, y = ark.test_qlinear(t(codes), t(scale), t(zp), W, use_gemm)
    qw, sw = oracle.prep_weight(w)
    for b in range(B):
        acc_o = oracle.matmul_integer(codes[b], zp[b], qw)
        y_o = oracle.dequant(acc_o, scale[b], sw, bias)
        assert np.array_equal(host(acc)[b * R:(b + 1) * R], acc_o.astype(np.int32))
        assert np.array_equal(host(y)[b * R:(b + 1) * R], y_o)


@pytest.mark.parametrize("V", [1003, 4096])
def test_masked_argmax_small_vocabularies(V):
    """A vocabulary that is not a multiple of 4 (the element-wise scan) and
    one that is (16-byte groups), with ties across groups and masked ids."""
    rng = np.random.default_rng(V)
    mask = (rng.random(V) < 0.1).astype(np.uint8)
    lg = rng.standard_normal((3, V)).astype(np.float32)
    lg[0, [3, 4, V - 2]] = 9.0                        # tie across groups -> id 3
    lg[1, :] = 2.0                                    # all equal -> first unmasked id
    lg[2, np.nonzero(mask == 0)[0][-1]] = 7.0         # maximum at the last unmasked id
    out = torch.empty(3, dtype=torch.int32, device=DEV)
    ark.masked_argmax(t(lg), t(mask), out)
    assert host(out).tolist() == oracle.masked_argmax(lg, mask).tolist()


def test_masked_argmax_bit_exact_and_forced_cases():
    V = 151936
    mask = synth.CONFIGS["c1"].mask()
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((6, V)).astype(np.float32)
    lg[0, V - 1] = 50.0                              # masked raw maximum
    lg[1, synth.CONFIGS["c1"].end_id] = 50.0         # the end id may win
    lg[2, 100] = lg[2, 7] = 60.0                     # tie -> lowest id
    lg[3, :] = np.nan
    lg[3, 12345] = -1.0                              # NaN never chosen
    lg[4, :V - 64] = np.nan                          # only masked/end ids left
    lg[5, :] = -np.inf
    out = torch.empty(6, dtype=torch.int32, device=DEV)
    ark.masked_argmax(t(lg), t(mask), out)
    assert host(out).tolist() == oracle.masked_argmax(lg, mask).tolist()
    assert host(out).tolist()[:5] == [int(np.argmax(np.where(mask == 1, -np.inf, lg[0]))),
                                      synth.CONFIGS["c1"].end_id, 7, 12345,
                                      synth.CONFIGS["c1"].end_id]


def test_cache_write_bit_exact():
    cfg = synth.SMALL.with_(batch=3)
    rng = np.random.default_rng(6)
    L, B, T, S = cfg.n_layers, 3, cfg.max_total_len, 5
    kc = [rng.standard_normal((B, T, 2, 128)).astype(np.float32) for _ in range(L)]
    vc = [rng.standard_normal((B, T, 2, 128)).astype(np.float32) for _ in range(L)]
    kd = rng.standard_normal((L, B, S, 2, 128)).astype(np.float32)
    vd = rng.standard_normal((L, B, S, 2, 128)).astype(np.float32)
    pos = [0, 17, T - S]
    gk, gv = [t(c) for c in kc], [t(c) for c in vc]
    ark.cache_write(ark.dims_of(cfg), pos, gk, gv, t(kd), t(vd))
    for l in range(L):
        assert np.array_equal(host(gk[l]), oracle.cache_write(kc[l], kd[l], pos))
        assert np.array_equal(host(gv[l]), oracle.cache_write(vc[l], vd[l], pos))


def test_embed_splice_bit_exact():
    cfg = synth.SMALL.with_(batch=2)
    table = synth.embed_table_f16(cfg)
    ids = synth.prompt_ids(cfg)
    audio = synth.audio_rows(cfg)
    out = torch.empty((2, cfg.prefill_len, cfg.hidden), dtype=torch.float32, device=DEV)
    ark.embed_splice(ark.dims_of(cfg), t(ids), t(table.view(np.int16)), t(audio),
                     cfg.audio_offset, out)
    assert np.array_equal(host(out), oracle.embed_splice(table, ids, audio, cfg.audio_offset))


@pytest.mark.gpu
def test_swiglu_elementwise_over_every_range():
    """The gate the GEMM epilogues compute (t = e^-|g| with a clamped
    argument, a reciprocal on [1, 2]) against the oracle's plain
    g / (1 + exp(-g)) * u: the working range, both underflow edges of e^-|g|,
    |g| near 0, fp32 subnormals and extremes, infinities and NaN.  The values
    are within 2.5e-7 (or one subnormal step) everywhere and bit-identical in
    all but a handful of cases (both are a few fp64 ulp from exact).  u is
    finite or NaN: with u infinite and -746 < g < -709.8 the oracle's
    e^-g overflows and yields NaN where the exact value is infinite."""
    rng = np.random.default_rng(11)
    sign = lambda n: np.where(rng.random(n) < 0.5, -1.0, 1.0)  # noqa: E731
    special = np.array([0.0, -0.0, 1e-45, -1e-45, 1.17e-38, -1.17e-38, np.inf, -np.inf, np.nan,
                        3.4e38, -3.4e38, 88.7, -88.7, 103.9, -103.9, 745.1, -745.1, 746.0,
                        -746.0, 800.0, -800.0])
    g = np.concatenate([
        rng.uniform(-30, 30, 200_000),
        rng.uniform(-760, -700, 20_000), rng.uniform(700, 760, 20_000),
        rng.uniform(-1e-3, 1e-3, 20_000),
        sign(40_000) * 10.0 ** rng.uniform(-45, 38.5, 40_000),
        np.repeat(special, 16)]).astype(np.float32)
    u = (rng.standard_normal(g.size) * 10.0 ** rng.uniform(-3, 3, g.size)).astype(np.float32)
    u[-16 * special.size::16] = 1.0
    u[-16 * special.size + 1::16] = -0.0
    u[-16 * special.size + 2::16] = 3e38
    u[-16 * special.size + 3::16] = np.nan
    y = host(ark.test_swiglu(torch.from_numpy(g).cuda(), torch.from_numpy(u).cuda()))
    with np.errstate(all="ignore"):
        yo = oracle.swiglu(g, u)
    assert np.array_equal(np.isnan(y), np.isnan(yo))
    fin = np.isfinite(yo)
    assert np.array_equal(y[~fin & ~np.isnan(yo)], yo[~fin & ~np.isnan(yo)])
    d = np.abs(y[fin].astype(np.float64) - yo[fin])
    assert np.all((d <= 2.5e-7 * np.abs(yo[fin])) | (d <= 1.5e-45))
    same = (y.view(np.uint32) == yo.view(np.uint32)) | (np.isnan(y) & np.isnan(yo))
    assert np.count_nonzero(~same) <= 3, np.nonzero(~same)[0][:10]


# M >= 128 takes the large-tile GEMM, whose epilogue also yields the
# per-sequence range (sequence boundaries inside a wave's rows, and many
# short sequences per wave); the others take a separate range pass
@pytest.mark.parametrize("B,R,n,k", [(3, 101, 200, 2048), (2, 200, 130, 1024), (40, 4, 96, 512),
                                     (1, 128, 64, 256), (4, 8, 96, 1024), (2, 30, 70, 2048),
                                     (2, 300, 8000, 256), (2, 100, 100, 192), (3, 400, 600, 1024)])
def test_gate_up_swiglu_and_sequence_range(B, R, n, k):
    rng = np.random.default_rng(7 * n + k + B * R)
    wg = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    wu = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    codes = rng.integers(0, 256, (B, R, k)).astype(np.uint8)
    scale = rng.uniform(0.001, 0.05, B).astype(np.float32)
    zp = rng.integers(0, 256, B).astype(np.uint8)
    G = ark.QLinear.from_f32(t(wg))
    U = ark.QLinear.from_f32(t(wu))
    y, lo, hi = ark.test_gate_up(t(codes), t(scale), t(zp), G, U)
    y, lo, hi = host(y), host(lo), host(hi)
    qg, sg = oracle.prep_weight(wg)
    qu, su = oracle.prep_weight(wu)
    for b in range(B):
        g = oracle.qlinear(codes[b], scale[b], zp[b], qg, sg)
        u = oracle.qlinear(codes[b], scale[b], zp[b], qu, su)
        yb = y[b * R:(b + 1) * R]
        # the products are exact; only exp may differ in its last fp64 bit
        np.testing.assert_allclose(yb, oracle.swiglu(g, u), rtol=2.5e-7, atol=0)
        # the range is exactly that of the values written
        assert lo[b] == yb.min() and hi[b] == yb.max()


# S > 1: the fp64 matrix-core kernel (range from its epilogue); S = 1: the
# split decode kernel and a separate range pass
@pytest.mark.parametrize("B,S,T,pos", [(2, 37, 512, (0, 300)), (3, 20, 64, (44, 0, 10)),
                                       (1, 1, 512, (100,)), (2, 1, 1024, (0, 1023)),
                                       (3, 1, 512, (31, 32, 511)), (4, 1, 64, (0, 63, 5, 33)),
                                       (1, 70, 128, (58,)),
                                       # a prefill that fills the cache, its key chunks split
                                       (1, 128, 128, (0,))])
def test_attention_and_sequence_range(B, S, T, pos):
    NH, NKV, D = 16, 2, 128
    rng = np.random.default_rng(B * 1000 + S * 10 + T)
    q = rng.standard_normal((B, S, NH * D)).astype(np.float32)
    kc = rng.standard_normal((B, T, NKV, D)).astype(np.float32)
    vc = rng.standard_normal((B, T, NKV, D)).astype(np.float32)
    kd = rng.standard_normal((B, S, NKV, D)).astype(np.float32)
    vd = rng.standard_normal((B, S, NKV, D)).astype(np.float32)
    out, lo, hi = ark.test_attention(t(q), t(kc), t(vc), t(kd), t(vd), pos, NKV)
    out, lo, hi = host(out), host(lo), host(hi)
    for b in range(B):
        kh = oracle.cache_write(kc[b:b + 1], kd[b:b + 1], np.array(pos[b:b + 1]))[0]
        vh = oracle.cache_write(vc[b:b + 1], vd[b:b + 1], np.array(pos[b:b + 1]))[0]
        ref = oracle.attention(q[b].reshape(S, NH, D), kh, vh, int(pos[b]))
        ob = out[b * S:(b + 1) * S]
        np.testing.assert_allclose(ob, ref, rtol=1e-5, atol=1e-6)
        assert lo[b] == ob.min() and hi[b] == ob.max()
