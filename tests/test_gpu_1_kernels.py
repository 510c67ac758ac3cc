"""Kernel-level parity: each HIP kernel family through its C-ABI entry point,
against the oracle's building blocks on the same seeded inputs."""
import math

import numpy as np
import pytest

import oracle as O
from s1_workloads import f32_to_bf16_bits
from tests.gpu_util import dev, dev_bits, host_bits, log, rel_l2, require_gpu, stream_ptr

pytestmark = pytest.mark.gpu

import prefill_only_decision_amd as s1  # noqa: E402
from prefill_only_decision_amd import binding as B  # noqa: E402


def _bits(rng, shape, scale=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("M,N,K,split", [
    (1, 64, 64, 1), (77, 130, 520, 1), (512, 6160, 2560, 1), (512, 2560, 9728, 3),
    (1000, 2560, 2048, 2), (129, 19456, 2560, 1), (2048, 3072, 2560, 1),
])
def test_gemm_bf16(M, N, K, split):
    torch = require_gpu()
    log(f"gemm bf16 M={M} N={N} K={K} split={split}")
    rng = np.random.default_rng([M, N, K])
    A, W = _bits(rng, (M, K)), _bits(rng, (N, K), 0.05)
    dA, dW = dev_bits(A), dev_bits(W)
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    B.gemm(B.S1_BF16, dA.data_ptr(), dW.data_ptr(), dC.data_ptr(), M, N, K, split, stream_ptr())
    torch.cuda.synchronize()
    ref = O.bf16_bits_to_float(A) @ O.bf16_bits_to_float(W).T
    C = dC.cpu().numpy()
    assert np.isfinite(C).all()
    assert rel_l2(C, ref) < 1e-5
    assert np.abs(C - ref).max() <= 1e-4 * np.abs(ref).max() + 1e-6


@pytest.mark.parametrize("M,N,K,split", [
    (1, 64, 64, 1), (300, 520, 640, 1), (300, 520, 640, 3), (4100, 264, 128, 1), (130, 2560, 9728, 4),
])
def test_gemm_bf16_every_tile_config(M, N, K, split):
    """Each tile configuration, on ragged M and N (partial tiles in both),
    several K tiles and K splits, against float64 products of the same bf16
    operands."""
    torch = require_gpu()
    rng = np.random.default_rng([M, N, K, 7])
    A, W = _bits(rng, (M, K)), _bits(rng, (N, K), 0.05)
    dA, dW = dev_bits(A), dev_bits(W)
    ref = O.bf16_bits_to_float(A) @ O.bf16_bits_to_float(W).T
    for cfg in range(B.gemm_tile_configs()):
        log(f"gemm bf16 cfg={cfg} M={M} N={N} K={K} split={split}")
        dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        B.gemm_cfg(B.S1_BF16, dA.data_ptr(), dW.data_ptr(), dC.data_ptr(), M, N, K, split, cfg, stream_ptr())
        torch.cuda.synchronize()
        C = dC.cpu().numpy()
        assert np.isfinite(C).all(), cfg
        assert rel_l2(C, ref) < 1e-5, cfg
        assert np.abs(C - ref).max() <= 1e-4 * np.abs(ref).max() + 1e-6, cfg


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (77, 200, 192), (300, 2560, 512), (1300, 2560, 256),
                                   (70, 5120, 128)])
def test_gemm_resid_norm(M, N, K):
    """The residual projection that leaves its RMSNorm to the next GEMM
    (s1k_gemm_resid_norm), in every tile configuration and with a K split:
    x += A W^T against float64 products of the same operands; rs * x against
    the oracle's rms_norm of the same updated x (gain 1) element by element;
    hb bitwise the updated x rounded to bf16 (without a K split) or x * rs
    rounded (with one); without a K split, rs bitwise the same in every
    configuration and for a row whatever M (one summation order, whatever the
    tile widths), N ragged against the tiles."""
    torch = require_gpu()
    rng = np.random.default_rng([M, N, K, 11])
    A, W = _bits(rng, (M, K)), _bits(rng, (N, K), 0.05)
    x0 = rng.standard_normal((M, N)).astype(np.float32)
    eps = 1e-6
    dA, dW = dev_bits(A), dev_bits(W)
    ref = x0.astype(np.float64) + O.bf16_bits_to_float(A) @ O.bf16_bits_to_float(W).T
    runs = [(cfg, 1) for cfg in [-1] + list(range(B.gemm_tile_configs()))]
    if N % 4 == 0 and K % 64 == 0 and K >= 128:
        runs += [(-1, 2), (1, 2)]
    first = None
    for cfg, split in runs:
        log(f"gemm resid norm cfg={cfg} split={split} M={M} N={N} K={K}")
        dx = dev(x0.copy())
        dh = torch.zeros((M, N), dtype=torch.int16, device="cuda")
        drs = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        form = B.gemm_resid_norm(dA.data_ptr(), dW.data_ptr(), dx.data_ptr(), M, N, K, split, cfg, eps,
                                 dh.data_ptr(), drs.data_ptr(), stream_ptr())
        torch.cuda.synchronize()
        x, hb, rs = dx.cpu().numpy(), host_bits(dh), drs.cpu().numpy()
        # without a K split the rows and their scales; an explicit configuration splits as asked
        if split == 1 or cfg >= 0:
            assert form == (2 if split == 1 else 1), (cfg, split, form)
        assert np.isfinite(x).all() and np.isfinite(rs).all(), (cfg, split)
        assert np.abs(x - ref).max() <= 1e-4 * np.abs(ref).max() + 1e-6, (cfg, split)
        want_hb = x if form == 2 else (x * rs[:, None]).astype(np.float32)
        assert np.array_equal(hb, f32_to_bf16_bits(want_hb)), (cfg, split)
        want = O.rms_norm(x.astype(np.float64), np.ones(N), eps)
        got = x.astype(np.float64) * rs[:, None].astype(np.float64)
        assert np.abs(got - want).max() <= 4e-6 * np.abs(want).max(), (cfg, split)
        if form == 2:
            if first is None:
                first = rs.copy()
            assert np.array_equal(rs.view(np.uint32), first.view(np.uint32)), (cfg, "rs differs between configurations")
    if M > 1:   # the first rows alone
        m2 = M // 2
        dx = dev(x0[:m2].copy())
        dh = torch.zeros((m2, N), dtype=torch.int16, device="cuda")
        drs = torch.zeros((m2,), dtype=torch.float32, device="cuda")
        B.gemm_resid_norm(dA.data_ptr(), dW.data_ptr(), dx.data_ptr(), m2, N, K, 1, -1, eps, dh.data_ptr(),
                          drs.data_ptr(), stream_ptr())
        torch.cuda.synchronize()
        assert np.array_equal(drs.cpu().numpy().view(np.uint32), first[:m2].view(np.uint32)), "rs depends on M"


@pytest.mark.parametrize("M,N,K,split", [
    (128, 1408, 256, 1), (100, 256, 688, 3), (5, 772, 256, 1), (77, 132, 100, 2), (33, 65, 36, 1),
    (600, 1000, 256, 1), (2100, 2100, 64, 1),
])
def test_gemm_f32(M, N, K, split):
    """fp32 GEMMs: the shape's own choice (the few-tile kernel with the K
    range split over waves, and over workgroups up to `split`; the 128 x 128
    kernel for many tiles) and configuration 0, on ragged
    M, N and K, against float64 products."""
    torch = require_gpu()
    rng = np.random.default_rng([M, N, K, 32])
    A = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    dA, dW = dev(A), dev(W)
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    for cfg in (None, 0):
        log(f"gemm f32 M={M} N={N} K={K} split={split} cfg={cfg}")
        dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        if cfg is None:
            B.gemm(B.S1_F32, dA.data_ptr(), dW.data_ptr(), dC.data_ptr(), M, N, K, split, stream_ptr())
        else:
            B.gemm_cfg(B.S1_F32, dA.data_ptr(), dW.data_ptr(), dC.data_ptr(), M, N, K, split, cfg, stream_ptr())
        torch.cuda.synchronize()
        C = dC.cpu().numpy()
        assert np.isfinite(C).all(), cfg
        assert rel_l2(C, ref) < 1e-5, cfg


def test_gemm_split_is_deterministic():
    torch = require_gpu()
    rng = np.random.default_rng(9)
    M, N, K = 512, 2560, 9728
    dA, dW = dev_bits(_bits(rng, (M, K))), dev_bits(_bits(rng, (N, K), 0.05))
    outs = []
    for _ in range(3):
        dC = torch.empty((M, N), dtype=torch.float32, device="cuda")
        B.gemm(B.S1_BF16, dA.data_ptr(), dW.data_ptr(), dC.data_ptr(), M, N, K, 3, stream_ptr())
        torch.cuda.synchronize()
        outs.append(dC.cpu().numpy())
    assert all(np.array_equal(outs[0], h) for h in outs[1:])


def _host_frag_pack(W, N, K):
    """Fragment order written out with numpy: block (nb, ks) holds, for lane
    l = 32 h + r, row 32 nb + r and columns 16 ks + 8 h .. + 7."""
    nb = (N + 31) // 32
    Wp = np.zeros((nb * 32, K), dtype=W.dtype)
    Wp[:N] = W
    return Wp.reshape(nb, 32, K // 16, 2, 8).transpose(0, 2, 3, 1, 4).reshape(-1)


@pytest.mark.parametrize("M,N,K", [
    (1, 64, 64), (77, 6160, 2560), (512, 19456, 2560), (300, 1000, 640), (130, 2560, 9728), (1000, 520, 128),
])
def test_gemm_wfrag(M, N, K):
    """The weight-direct GEMM over a fragment-packed weight: the packing
    against numpy, the product against float64 products of the same bf16
    operands, and bitwise equality with the LDS-staged kernel without a K
    split (same matrix instructions in the same K order)."""
    torch = require_gpu()
    log(f"gemm wfrag M={M} N={N} K={K}")
    rng = np.random.default_rng([M, N, K, 11])
    A, W = _bits(rng, (M, K)), _bits(rng, (N, K), 0.05)
    dA, dW = dev_bits(A), dev_bits(W)
    nbytes = B.frag_bytes(N, K)
    assert nbytes == (N + 31) // 32 * 32 * K * 2
    dWf = torch.full((nbytes // 2,), -1, dtype=torch.int16, device="cuda")
    B.frag_pack(dW.data_ptr(), N, K, False, dWf.data_ptr(), stream_ptr())
    dR = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    B.gemm_cfg(B.S1_BF16, dA.data_ptr(), dW.data_ptr(), dR.data_ptr(), M, N, K, 1, 1, stream_ptr())
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dWf), _host_frag_pack(W, N, K))
    ref = O.bf16_bits_to_float(A) @ O.bf16_bits_to_float(W).T
    R = dR.cpu().numpy()
    for tile in (1, 2, 3, 4):
        dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        B.gemm_wfrag(dA.data_ptr(), dWf.data_ptr(), dC.data_ptr(), M, N, K, False, tile=tile, stream=stream_ptr())
        torch.cuda.synchronize()
        C = dC.cpu().numpy()
        assert np.isfinite(C).all(), tile
        assert rel_l2(C, ref) < 1e-5, tile
        assert np.abs(C - ref).max() <= 1e-4 * np.abs(ref).max() + 1e-6, tile
        assert np.array_equal(C, R), tile


@pytest.mark.parametrize("M,F,K", [(512, 9728, 2560), (77, 96, 640), (1, 32, 64), (700, 160, 128)])
def test_gemm_wfrag_swiglu(M, F, K):
    """Gate/up rows stored as the decoder stores them ([32 gate | 32 up] per
    64 rows), packed with the 16-row interleave, through the SwiGLU epilogue
    of the weight-direct GEMM: silu(x Wg^T) * (x Wu^T) within bf16 rounding
    of the float64 result."""
    torch = require_gpu()
    log(f"gemm wfrag swiglu M={M} F={F} K={K}")
    rng = np.random.default_rng([M, F, K, 12])
    A = _bits(rng, (M, K))
    Wg, Wu = _bits(rng, (F, K), 0.05), _bits(rng, (F, K), 0.05)
    W = np.zeros((2 * F, K), dtype=np.uint16)
    i = np.arange(F)
    W[64 * (i // 32) + i % 32] = Wg
    W[64 * (i // 32) + i % 32 + 32] = Wu
    dA, dW = dev_bits(A), dev_bits(W)
    dWf = torch.empty((B.frag_bytes(2 * F, K) // 2,), dtype=torch.int16, device="cuda")
    B.frag_pack(dW.data_ptr(), 2 * F, K, True, dWf.data_ptr(), stream_ptr())
    a = O.bf16_bits_to_float(A)
    g, u = a @ O.bf16_bits_to_float(Wg).T, a @ O.bf16_bits_to_float(Wu).T
    ref = g / (1 + np.exp(-g)) * u
    outs = []
    for tile in (1, 2, 3, 4):
        dH = torch.full((M, F), -1, dtype=torch.int16, device="cuda")
        B.gemm_wfrag(dA.data_ptr(), dWf.data_ptr(), dH.data_ptr(), M, 2 * F, K, True, tile=tile, stream=stream_ptr())
        torch.cuda.synchronize()
        H = O.bf16_bits_to_float(host_bits(dH))
        assert np.isfinite(H).all(), tile
        assert (np.abs(H - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * np.abs(ref).max()).all(), tile
        assert rel_l2(H, ref) < 4e-3, tile
        outs.append(H)
    assert all(np.array_equal(outs[0], h) for h in outs[1:])


@pytest.mark.parametrize("dtype", [B.S1_BF16, B.S1_F32])
def test_rmsnorm_and_embed(dtype):
    torch = require_gpu()
    rng = np.random.default_rng(dtype + 3)
    T, d, V = 37, 2560, 1000
    x = (rng.standard_normal((T, d)) * 3).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    out = torch.empty((T, d), dtype=torch.int16 if dtype == B.S1_BF16 else torch.float32, device="cuda")
    dx, dw = dev(x), dev(w)
    B.rmsnorm(dtype, dx.data_ptr(), dw.data_ptr(), out.data_ptr(), T, d, 1e-6, stream_ptr())
    torch.cuda.synchronize()
    ref = O.rms_norm(x.astype(np.float64), w.astype(np.float64), 1e-6)
    got = O.bf16_bits_to_float(host_bits(out)) if dtype == B.S1_BF16 else out.cpu().numpy()
    tol = 2.0 ** -8 if dtype == B.S1_BF16 else 1e-6
    assert (np.abs(got - ref) <= tol * np.abs(ref) + 1e-7).all()
    # embedding gather is a copy: exact
    if dtype == B.S1_BF16:
        E = _bits(rng, (V, d), 0.02)
        dE = dev_bits(E)
        Ef = O.bf16_bits_to_float(E)
    else:
        Ef = (rng.standard_normal((V, d)) * 0.02).astype(np.float32)
        dE = dev(Ef)
    ids = rng.integers(0, V, T).astype(np.int32)
    dx2 = torch.empty((T, d), dtype=torch.float32, device="cuda")
    dids = dev(ids)
    B.embed(dtype, dids.data_ptr(), dE.data_ptr(), dx2.data_ptr(), T, d, stream_ptr())
    torch.cuda.synchronize()
    assert np.array_equal(dx2.cpu().numpy(), np.asarray(Ef)[ids].astype(np.float32))


def test_lora_merge_bf16():
    torch = require_gpu()
    rng = np.random.default_rng(11)
    out_dim, in_dim, r = 300, 2560, 32
    W, A, Bm = _bits(rng, (out_dim, in_dim), 0.02), _bits(rng, (r, in_dim), 0.02), _bits(rng, (out_dim, r), 0.02)
    dW, dA, dB = dev_bits(W), dev_bits(A), dev_bits(Bm)
    dO = torch.empty((out_dim, in_dim), dtype=torch.int16, device="cuda")
    B.lora_merge(B.S1_BF16, dW.data_ptr(), dA.data_ptr(), dB.data_ptr(), dO.data_ptr(), out_dim, in_dim, r,
                 2.0, stream_ptr())
    torch.cuda.synchronize()
    got = host_bits(dO).astype(np.int64)
    f = O.bf16_bits_to_float
    ref = O.round_to_bf16_bits(O.lora_merge(f(W), f(A), f(Bm), 64.0, 32)).astype(np.int64)
    diff = np.abs(got - ref)
    assert diff.max() <= 1, diff.max()
    assert (diff > 0).mean() < 1e-3
    # no adapter: exact copy
    B.lora_merge(B.S1_BF16, dW.data_ptr(), 0, 0, dO.data_ptr(), out_dim, in_dim, r, 2.0, stream_ptr())
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dO), W)


def _elementwise_excess(got, ref, floor=1e-4):
    """Largest |got - ref| over its bound, per (row, head): one bf16 rounding
    of the result (2^-8 |ref|: half an ulp, or a full one when the kernel's
    fp32 value sits on the other side of a rounding boundary) plus floor x
    the row-head's RMS for fp32 accumulation.  <= 1 passes; a bad row or
    head shows up as >> 1 even when the norm over the whole tensor is small."""
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True)) + 1e-30
    bound = 2.0 ** -8 * np.abs(ref) + floor * rms
    return float((np.abs(np.asarray(got, np.float64) - ref) / bound).max()) if ref.size else 0.0


def _scan_case(H, lens, seed, with_init=True, chunked=False):
    torch = require_gpu()
    rng = np.random.default_rng(seed)
    T, dk = int(sum(lens)), 128
    qkv = _bits(rng, (T, 3 * H * dk), 1.0)
    lg = np.log(1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = len(lens)
    s0 = (rng.standard_normal((n, H, dk, dk)) * 0.1).astype(np.float32) if with_init else None
    d_qkv, d_lg = dev_bits(qkv), dev(lg)
    d_o = torch.zeros((T, H * dk), dtype=torch.int16, device="cuda")
    d_s0 = dev(s0) if with_init else None
    d_sf = torch.zeros((n, H, dk, dk), dtype=torch.float32, device="cuda")
    base = d_qkv.data_ptr()
    if chunked:
        B.la_scan_chunked(base, base + 2 * H * dk, base + 4 * H * dk, 3 * H * dk, d_lg.data_ptr(),
                          d_o.data_ptr(), T, H, cu, d_s0.data_ptr() if with_init else None,
                          d_sf.data_ptr(), stream_ptr())
    else:
        B.la_scan(B.S1_BF16, base, base + 2 * H * dk, base + 4 * H * dk, 3 * H * dk, d_lg.data_ptr(),
                  d_o.data_ptr(), T, H, dk, dk, cu, d_s0.data_ptr() if with_init else None,
                  d_sf.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
    o = O.bf16_bits_to_float(host_bits(d_o)).reshape(T, H, dk)
    sf = d_sf.cpu().numpy()
    qkvf = O.bf16_bits_to_float(qkv).reshape(T, 3, H, dk)
    worst_o = worst_s = worst_raw = worst_el = 0.0
    for i in range(n):
        a, b = cu[i], cu[i + 1]
        ro, rs = O.la_scan_unrolled(qkvf[a:b, 0], qkvf[a:b, 1], qkvf[a:b, 2], np.exp(lg[a:b].astype(np.float64)),
                                    s0[i].astype(np.float64) if with_init else None)
        if b > a:
            # the kernel rounds o once to bf16 at the end; everything before is
            # exact products with fp32 accumulation
            worst_o = max(worst_o, rel_l2(o[a:b], O.bf16_bits_to_float(O.round_to_bf16_bits(ro))))
            worst_raw = max(worst_raw, rel_l2(o[a:b], ro))
            worst_el = max(worst_el, _elementwise_excess(o[a:b], ro))
        worst_s = max(worst_s, rel_l2(sf[i], rs))
        if with_init or b > a:
            assert np.abs(sf[i] - rs).max() <= 1e-5 * np.abs(rs).max() + 1e-30, i
    log(f"scan{' (chunked)' if chunked else ''} H={H} lens={lens}: rel L2 o vs rounded oracle {worst_o:.2e} (vs unrounded {worst_raw:.2e}), "
        f"state {worst_s:.2e}, element-wise excess {worst_el:.2f}")
    assert worst_o < 1e-3 and worst_s < 1e-5 and worst_el <= 1.0


@pytest.mark.parametrize("H,lens", [
    (16, [1, 63, 64, 65, 200]),            # 80 chains: 1 wave per workgroup
    (32, [130, 7, 64, 255]),               # 128 chains: 2 waves
    (64, [1, 100, 64, 300]),               # 256 chains: 4 waves
])
def test_scan_bf16(H, lens):
    _scan_case(H, lens, seed=H)


def test_scan_bf16_zero_init_and_empty_sequence():
    _scan_case(16, [0, 40, 0, 129], seed=5, with_init=False)


@pytest.mark.parametrize("H,lens,init", [
    (16, [512], True), (16, [1, 63, 64, 65, 200, 0], True), (4, [4096], False), (40, [300, 33], True),
])
def test_scan_bf16_chunk_parallel(H, lens, init):
    _scan_case(H, lens, seed=H + len(lens), with_init=init, chunked=True)


@pytest.mark.parametrize("H,dk,dv,lens", [
    (4, 64, 64, [1, 50, 77]), (2, 128, 128, [0, 33, 300]), (3, 128, 64, [512, 31]), (2, 64, 128, [600, 5]),
])
def test_scan_f32(H, dk, dv, lens):
    """fp32 scan against the float64 recurrence, with initial and final
    states: batches whose longest sequence has at most 512 tokens run the
    whole-sequence kernel (one chunk per sequence, all rows in parallel),
    longer ones the sequential chunked kernel; an empty sequence passes its
    initial state through."""
    torch = require_gpu()
    log(f"scan f32 H={H} dk={dk} dv={dv} lens={lens}")
    rng = np.random.default_rng([21, H, dk, dv, len(lens)])
    T = sum(lens)
    n = len(lens)
    ld = H * (2 * dk + dv)
    qkv = rng.standard_normal((T, ld)).astype(np.float32)
    lg = np.log(1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    s0 = rng.standard_normal((n, H, dk, dv)).astype(np.float32)
    d_qkv, d_lg, d_s0 = dev(qkv), dev(lg), dev(s0)
    d_o = torch.zeros((T, H * dv), dtype=torch.float32, device="cuda")
    d_sf = torch.zeros_like(d_s0)
    base = d_qkv.data_ptr()
    B.la_scan(B.S1_F32, base, base + 4 * H * dk, base + 8 * H * dk, ld, d_lg.data_ptr(), d_o.data_ptr(),
              T, H, dk, dv, cu, d_s0.data_ptr(), d_sf.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
    x = qkv.astype(np.float64)
    qa = x[:, :H * dk].reshape(T, H, dk)
    ka = x[:, H * dk:2 * H * dk].reshape(T, H, dk)
    va = x[:, 2 * H * dk:].reshape(T, H, dv)
    out, sf = d_o.cpu().numpy().reshape(T, H, dv), d_sf.cpu().numpy()
    for i in range(n):
        a, b = cu[i], cu[i + 1]
        ro, rs = O.la_scan_recurrent(qa[a:b], ka[a:b], va[a:b], np.exp(lg[a:b].astype(np.float64)),
                                     s0[i].astype(np.float64))
        if b > a:
            assert rel_l2(out[a:b], ro) < 1e-5, i
        assert rel_l2(sf[i], rs) < 1e-5, i


def _attn_case(dtype, Hq, Hkv, hd, seqs, seed, block_rows=0, piece=0, shared=False):
    """seqs: list of (q_len, prefix_len).  shared: every sequence continues
    one prefix (the first sequence's prefix_len rows), as the branches of a
    request do."""
    torch = require_gpu()
    rng = np.random.default_rng(seed)
    Tq = sum(s[0] for s in seqs)
    Tp = sum(s[1] for s in seqs)
    Tkv = Tq + Tp
    if dtype == B.S1_BF16:
        q, k, v = _bits(rng, (Tq, Hq, hd)), _bits(rng, (Tkv, Hkv, hd)), _bits(rng, (Tkv, Hkv, hd))
        dq, dk_, dv_ = dev_bits(q), dev_bits(k), dev_bits(v)
        qf, kf, vf = (O.bf16_bits_to_float(a) for a in (q, k, v))
        do = torch.zeros((Tq, Hq, hd), dtype=torch.int16, device="cuda")
    else:
        qf, kf, vf = (rng.standard_normal(s).astype(np.float32) for s in ((Tq, Hq, hd), (Tkv, Hkv, hd), (Tkv, Hkv, hd)))
        dq, dk_, dv_ = dev(qf), dev(kf), dev(vf)
        do = torch.zeros((Tq, Hq, hd), dtype=torch.float32, device="cuda")
    q_row0, q_len, kv_row0, pre_row0, pre_len = [], [], [], [], []
    rq, rp = 0, Tq
    for (L, P) in seqs:
        q_row0.append(rq); q_len.append(L); kv_row0.append(rq); pre_row0.append(rp); pre_len.append(P)
        rq += L
        rp += 0 if shared else P
    B.attention(dtype, dq.data_ptr(), dk_.data_ptr(), dv_.data_ptr(), do.data_ptr(), Hq, Hkv, hd,
                q_row0, q_len, kv_row0, pre_row0, pre_len, stream_ptr(), block_rows=block_rows, piece=piece)
    torch.cuda.synchronize()
    got = O.bf16_bits_to_float(host_bits(do)) if dtype == B.S1_BF16 else do.cpu().numpy().astype(np.float64)
    worst = worst_el = 0.0
    grp = Hq // Hkv
    for i, (L, P) in enumerate(seqs):
        if L == 0:
            continue
        a = q_row0[i]
        kk = np.concatenate([kf[pre_row0[i]:pre_row0[i] + P], kf[a:a + L]]).astype(np.float64)
        vv = np.concatenate([vf[pre_row0[i]:pre_row0[i] + P], vf[a:a + L]]).astype(np.float64)
        ref = O.causal_attention(qf[a:a + L].astype(np.float64), kk, vv, P + np.arange(L), np.arange(P + L))
        worst = max(worst, rel_l2(got[a:a + L], ref))
        # element-wise: bf16 probabilities in the second product change each
        # output by at most 2^-9 max|v| (the weights sum to one), a normaliser
        # summed from them by at most 2^-9 |o|, and the bf16 output rounding
        # by 2^-9 |o|; fp32 paths: 1e-5 in place of 2^-9
        vmax = np.abs(vv).max(axis=(0, 2))[np.arange(Hq) // grp][None, :, None]
        unit = 2.0 ** -9 if dtype == B.S1_BF16 else 1e-5
        bound = unit * (vmax + 2.0 * np.abs(ref)) + 1e-6
        worst_el = max(worst_el, float((np.abs(got[a:a + L] - ref) / bound).max()))
    log(f"attention dtype={dtype} rows/workgroup={block_rows or 'auto'} piece={piece} shared={shared} "
        f"seqs={seqs}: rel L2 {worst:.2e}, element-wise excess {worst_el:.2f}")
    assert worst_el <= 1.0, worst_el
    return worst


@pytest.mark.parametrize("block_rows", [0, 32, 64, 128])
@pytest.mark.parametrize("seqs", [
    [(1, 0), (100, 0), (128, 0), (129, 0), (300, 0)],
    [(64, 200), (1, 70), (130, 4096)],
])
def test_attention_bf16(seqs, block_rows):
    assert _attn_case(B.S1_BF16, 16, 4, 128, seqs, seed=len(seqs), block_rows=block_rows) < 1e-2


@pytest.mark.parametrize("piece", [128, 256, -1])
@pytest.mark.parametrize("seqs", [
    [(1, 0), (100, 0), (128, 0), (129, 0), (300, 0), (512, 0)],
    [(64, 200), (1, 70), (130, 4096)],
])
def test_attention_bf16_split_keys(seqs, piece):
    """Keys cut into pieces run by separate workgroups and merged in order,
    against the same definition and element-wise bound."""
    assert _attn_case(B.S1_BF16, 16, 4, 128, seqs, seed=len(seqs) + 7, piece=piece) < 1e-2


@pytest.mark.parametrize("piece", [128, 1024, -1])
@pytest.mark.parametrize("P,lens", [(4096, [64] * 5), (100, [64, 1, 65, 130]), (257, [3, 200])])
def test_attention_bf16_shared_prefix(P, lens, piece):
    """Branches of one prefix: one sweep of the prefix keys for all their
    queries (prefix lengths off the 64-key grid included), merged with each
    branch's own causal keys."""
    seqs = [(L, P) for L in lens]
    assert _attn_case(B.S1_BF16, 16, 4, 128, seqs, seed=P + len(lens), piece=piece, shared=True) < 1e-2


def test_attention_bf16_gqa5():
    # 40 query heads over 8 kv heads (groups of 5)
    assert _attn_case(B.S1_BF16, 40, 8, 128, [(200, 0), (33, 17)], seed=40) < 1e-2


@pytest.mark.parametrize("Hq,Hkv,hd,seqs", [
    (4, 4, 64, [(1, 0), (70, 0), (20, 30)]), (8, 2, 128, [(130, 0), (17, 100), (64, 0)]),
])
def test_attention_f32(Hq, Hkv, hd, seqs):
    assert _attn_case(B.S1_F32, Hq, Hkv, hd, seqs, seed=3 + hd) < 1e-5


@pytest.mark.parametrize("dtype,d", [(B.S1_BF16, 2560), (B.S1_F32, 2560), (B.S1_BF16, 2568), (B.S1_BF16, 260)])
def test_readout(dtype, d):
    """Widths that are whole 16-byte chunks of bf16 (2560 = 5 x 512 values,
    2568 with a ragged last pass) take the wide-load option loop; 260 the
    8-byte one."""
    torch = require_gpu()
    rng = np.random.default_rng(31 + dtype + d)
    V, R = 1000, 20
    x = (rng.standard_normal((R, d)) * 5).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    if dtype == B.S1_BF16:
        E = _bits(rng, (V, d), 0.02)
        dE = dev_bits(E)
        Ef = O.bf16_bits_to_float(E)
    else:
        Ef = (rng.standard_normal((V, d)) * 0.02).astype(np.float32)
        dE = dev(Ef)
    Q = 40
    Ks = rng.integers(2, 41, Q)
    types = rng.integers(0, 3, Q).astype(np.uint8)
    Ks[types == 2] = 2
    Ks[0], types[0] = 300, 0                       # one wide question
    offs = np.concatenate([[0], np.cumsum(Ks)]).astype(np.int32)
    ids = np.concatenate([rng.choice(V, k, replace=False) for k in Ks]).astype(np.int32)
    ids[offs[5]:offs[6]] = ids[offs[5]]            # duplicate options: exact tie
    rows = rng.integers(0, R, Q).astype(np.int32)
    dx, dw = dev(x), dev(w)
    drows, doffs, dids, dtypes = dev(rows), dev(offs), dev(ids), dev(types)
    dp = torch.zeros(int(offs[-1]), dtype=torch.float32, device="cuda")
    dd = torch.zeros((Q, 6), dtype=torch.float32, device="cuda")
    B.readout(dtype, dx.data_ptr(), d, dw.data_ptr(), 1e-6, dE.data_ptr(), Q, drows.data_ptr(), doffs.data_ptr(),
              dids.data_ptr(), dtypes.data_ptr(), dp.data_ptr(), dd.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
    p = dp.cpu().numpy()
    dec = dd.cpu().numpy().copy().view(np.uint8).view(s1.DECISION_DTYPE).reshape(Q)
    for j in range(Q):
        rp, f = O.readout(x[rows[j]].astype(np.float64), w.astype(np.float64),
                          np.asarray(Ef, np.float64)[ids[offs[j]:offs[j + 1]]], 1e-6, int(types[j]))
        assert np.abs(p[offs[j]:offs[j + 1]] - rp).max() < 1e-4
        srt = np.sort(rp)
        if srt[-1] - srt[-2] > 1e-4 or j == 5:
            assert dec[j]["choice"] == f["choice"], j
        for key in ("score", "noul", "answer_confidence", "confidence", "entropy_confidence"):
            assert abs(float(dec[j][key]) - f[key]) < 1e-3 * max(1.0, abs(f[key])), (j, key)


@pytest.mark.parametrize("H,lens,init", [(4, [1, 64, 65, 200, 640], True), (2, [1100], False), (16, [512], False)])
def test_gdn_scan_bf16(H, lens, init):
    """Gated DeltaNet scan against the oracle's token-by-token recurrence on
    the same bf16 q, k, v (q and k unit vectors), gates and write strengths."""
    torch = require_gpu()
    log(f"gdn scan H={H} lens={lens} init={init}")
    rng = np.random.default_rng([H, len(lens), 7])
    T, dk = int(sum(lens)), 128
    qk = rng.standard_normal((T, 2, H, dk))
    qk = qk / np.linalg.norm(qk, axis=-1, keepdims=True)
    qkv = np.concatenate([qk.reshape(T, 2 * H * dk), rng.standard_normal((T, H * dk))], axis=1)
    bits = O.round_to_bf16_bits(qkv)
    g = 1.0 / (1.0 + np.exp(-(rng.standard_normal((T, H)) + 2.0)))
    lg = np.log(g).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = len(lens)
    s0 = (rng.standard_normal((n, H, dk, dk)) * 0.1).astype(np.float32) if init else None
    d_qkv, d_lg, d_b = dev_bits(bits), dev(lg), dev(beta)
    d_o = torch.zeros((T, H * dk), dtype=torch.int16, device="cuda")
    d_s0 = dev(s0) if init else None
    d_sf = torch.zeros((n, H, dk, dk), dtype=torch.float32, device="cuda")
    base = d_qkv.data_ptr()
    B.gdn_scan(base, base + 2 * H * dk, base + 4 * H * dk, 3 * H * dk, d_lg.data_ptr(), d_b.data_ptr(),
               d_o.data_ptr(), T, H, cu, d_s0.data_ptr() if init else None, d_sf.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
    o = O.bf16_bits_to_float(host_bits(d_o)).reshape(T, H, dk)
    sf = d_sf.cpu().numpy()
    x = O.bf16_bits_to_float(bits).reshape(T, 3, H, dk)
    worst_o = worst_s = worst_el = 0.0
    for i in range(n):
        a, b = cu[i], cu[i + 1]
        ro, rs = O.gdn_recurrent(x[a:b, 0], x[a:b, 1], x[a:b, 2], np.exp(lg[a:b].astype(np.float64)),
                                 beta[a:b].astype(np.float64), s0[i].astype(np.float64) if init else None)
        if b > a:
            worst_o = max(worst_o, rel_l2(o[a:b], O.bf16_bits_to_float(O.round_to_bf16_bits(ro))))
            worst_el = max(worst_el, _elementwise_excess(o[a:b], ro, floor=1e-3))
        worst_s = max(worst_s, rel_l2(sf[i], rs))
    log(f"  rel L2 o vs rounded token recurrence {worst_o:.2e}, state {worst_s:.2e}, "
        f"element-wise excess {worst_el:.2f}")
    assert worst_o < 1e-3 and worst_s < 1e-5 and worst_el <= 1.0


def test_peak_probes():
    """The achievable-peak probes behind the benchmark's measured fractions:
    the copy is exact (ragged length: past the last full group of four
    accesses per thread), the read leaves the sink untouched for data whose
    xor misses its pattern, and the matrix loop equals iters x 8 products of
    its operands on every lane of a tile."""
    torch = require_gpu()
    nbytes = (1 << 20) + 48
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    B.stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream_ptr())
    sink = torch.full((1024,), 7, dtype=torch.int32, device="cuda")
    B.stream_read(src.data_ptr(), nbytes, sink.data_ptr(), stream_ptr())
    # seed: A = all ones, B = all ones (bf16 0x3F80): each 32x32x16 product adds 16
    seed = torch.full((1024,), 0x3F80, dtype=torch.int16, device="cuda")
    out = torch.empty(2 * 256, dtype=torch.float32, device="cuda")
    B.mfma_peak(seed.data_ptr(), 2, 3, out.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert (sink == 7).all()
    # every lane sums 8 accumulators x 16 rows, each 3 x 16
    assert (out == 8 * 16 * 3 * 16).all()
