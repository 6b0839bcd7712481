"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: NF4 codes, 8-bit absmax codes, second-level scales, dequantized
bf16. Tolerance (fp32 outputs): relative Frobenius error <= 2e-3 and max
element error <= 1e-2 x RMS of the oracle output, for y, dX, dA, dB.
"""
import concurrent.futures as cf
import ctypes
import os
import types

import numpy as np
import pytest
import torch

import oracle
import qlora_fine_tuning_blockwise_amd as q
from qlora_fine_tuning_blockwise_amd import synthetic as syn

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REL_FROB = 2e-3
MAX_REL_RMS = 1e-2
POOL = cf.ThreadPoolExecutor(max_workers=8)  # oracle calls release the GIL


def say(*a):
    print(*a, flush=True)


def tol_check(got, ref, name):
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    nref = np.linalg.norm(ref)
    rf = np.linalg.norm(got - ref) / nref if nref > 0 else np.linalg.norm(got)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    mx = np.max(np.abs(got - ref)) if ref.size else 0.0
    assert rf <= REL_FROB, f"{name}: relative Frobenius error {rf:.3e}"
    assert mx <= MAX_REL_RMS * rms + 1e-30, f"{name}: max error {mx:.3e} vs rms {rms:.3e}"
    return rf


def dev_bf16(bits):
    return syn.bits_to_torch_bf16(bits).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def quantize_gpu(W, fmt=0):
    w = q.qlora_quantize_nf4_dq(W, dq_format=fmt)
    torch.cuda.synchronize()
    return w


def assert_nf4_equal(w, codes, q8, s2, name):
    gc, gq, gs = host(w.codes), host(w.absmax_q), host(w.absmax_scale)
    if not np.array_equal(gc, codes):
        i = int(np.argmax(gc != codes))
        raise AssertionError(f"{name}: codes differ first at byte {i}: {gc[i]:#x} vs {codes[i]:#x}")
    assert np.array_equal(gq, q8), f"{name}: absmax codes differ"
    assert np.array_equal(gs.view(np.uint32), s2.view(np.uint32)), f"{name}: scales differ"


# ------------------------------------------------------------------ quantize / dequant
def _edge_weights():
    """bf16 weights hitting the corners of the quantizer (64-aligned rows)."""
    lv, _ = oracle.nf4_codebook()
    rows = []
    rng = np.random.default_rng(99)
    for c in (1.0, 0.02, 3.0e38 / 2, 2.0 ** -70, 2.0 ** 70, 1e-39):
        rows.append((lv.astype(np.float64) * c).astype(np.float32))
        mids = ((lv[:-1].astype(np.float64) + lv[1:]) / 2 * c).astype(np.float32)
        rows.append(np.concatenate([mids, np.array([c], np.float32)]))
    rows.append(np.zeros(64, np.float32))
    rows.append(np.full(64, -0.0, np.float32))
    rows.append(np.array([1e-45, -1e-45, 1e-41, -2e-40, 0.0] * 13, np.float32)[:64])
    rows.append(np.full(64, 0.125, np.float32))
    rows.append(np.concatenate([rng.standard_normal(63).astype(np.float32) * 1e-3,
                                np.array([-7.0], np.float32)]))
    flat = np.concatenate([np.resize(r, 64) for r in rows])
    flat = np.concatenate([flat, rng.standard_normal(64 * 300).astype(np.float32) * 0.02])
    return syn.to_bf16_bits(flat).reshape(-1, 64)


@pytest.mark.parametrize("shape", [(1, 64), (3, 192), (5, 4096), (257, 640)])
def test_quantize_ragged_shapes_bit_exact(shape):
    say("quantize ragged", shape)
    Wb = syn.normal_bf16(shape, 0.02, 100 + shape[0])
    w = quantize_gpu(dev_bf16(Wb))
    assert_nf4_equal(w, *oracle.quantize_nf4_dq(Wb, "bf16"), f"ragged {shape}")


def test_quantize_edge_values_bit_exact():
    Wb = _edge_weights()
    say("quantize edge values", Wb.shape)
    w = quantize_gpu(dev_bf16(Wb))
    codes, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16")
    assert_nf4_equal(w, codes, q8, s2, "edge")
    deq = syn.torch_bf16_to_bits(q.qlora_dequant_bf16(w)).ravel()
    _, wb = oracle.dequant_dq(codes, q8, s2)
    assert np.array_equal(deq, wb)


def _near_threshold_rows():
    """Blocks whose quotients w/c1 sit within 4 bf16 steps of every decision
    threshold, for every 8-bit absmax significand at three scales and both
    signs of the absmax element: the cases where the code decision is closest."""
    _, thr = oracle.nf4_codebook()
    rows = []
    for e in (0, -40, 40):
        for m in range(128):
            c1_bits = np.uint16(((127 + e) << 7) | m)
            c1 = float(oracle.bf16_to_f32(np.array([c1_bits], np.uint16))[0])
            centre = syn.to_bf16_bits((thr.astype(np.float64) * c1).astype(np.float32))
            cand = (centre.astype(np.int32)[:, None] + np.arange(-4, 5)[None, :]).ravel()
            cand = cand.astype(np.uint16)
            for sign in (0, 0x8000):
                for k in range(0, cand.size, 63):
                    part = cand[k:k + 63]
                    row = np.zeros(64, np.uint16)
                    row[0] = c1_bits | sign
                    row[1:1 + part.size] = part
                    rows.append(row)
    return np.stack(rows)


def test_quantize_near_threshold_quotients_bit_exact():
    Wb = _near_threshold_rows()
    say("quantize near-threshold quotients", Wb.shape)
    w = quantize_gpu(dev_bf16(Wb))
    assert_nf4_equal(w, *oracle.quantize_nf4_dq(Wb, "bf16"), "near-threshold quotients")


def test_quantize_f32_linear_1024_bit_exact():
    cfg = syn.LINEAR_1024
    W = syn.normal_f32(cfg["weights"]["w"], cfg["w_std"], syn.seed_of(1, 0))
    say("quantize f32 1024x1024")
    w = quantize_gpu(torch.from_numpy(W).to(DEV))
    codes, q8, s2 = oracle.quantize_nf4_dq(W, "f32")
    assert_nf4_equal(w, codes, q8, s2, "f32 1024")
    deq = syn.torch_bf16_to_bits(q.qlora_dequant_bf16(w)).ravel()
    assert np.array_equal(deq, oracle.dequant_dq(codes, q8, s2)[1])


def test_quantize_f32_edge_values():
    rng = np.random.default_rng(5)
    W = np.concatenate([rng.standard_normal(64 * 40).astype(np.float32) * 0.02,
                        np.array([1e-40, -3e-39, 0.0, 1e30] * 16, np.float32),
                        np.zeros(64, np.float32)]).reshape(-1, 64)
    w = quantize_gpu(torch.from_numpy(W).to(DEV))
    assert_nf4_equal(w, *oracle.quantize_nf4_dq(W, "f32"), "f32 edge")


@pytest.mark.parametrize("name", ["q", "up"])
def test_quantize_dequant_llama7b_bit_exact(name):
    shape = syn.LLAMA7B_TRAIN["weights"][name]
    say("quantize llama7b", name, shape)
    W = syn.torch_normal_bf16(shape, 0.02, syn.seed_of(2, 0 if name == "q" else 1), DEV)
    w = quantize_gpu(W)
    Wb = syn.torch_bf16_to_bits(W)
    codes, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16")
    assert_nf4_equal(w, codes, q8, s2, name)
    deq = syn.torch_bf16_to_bits(q.qlora_dequant_bf16(w)).ravel()
    assert np.array_equal(deq, oracle.dequant_dq(codes, q8, s2)[1])


def _sample_groups(ng, k, seed):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(ng, size=min(k, ng), replace=False).tolist()) | {0, ng - 1}
    return sorted(pick)


def test_quantize_70b_layer_sampled_groups():
    """All 7 projections of the 70B-shaped layer; the oracle checks 48 sampled
    16384-weight groups per projection (groups are independent)."""
    cfg = syn.LAYER_70B
    for i, (name, shape) in enumerate(cfg["weights"].items()):
        say("quantize 70b", name, shape)
        W = syn.torch_normal_bf16(shape, cfg["w_std"], syn.seed_of(4, i), DEV)
        w = quantize_gpu(W)
        flat = W.view(-1)
        n = flat.numel()
        ng = (n // 64 + 255) // 256
        gc, gq, gs = host(w.codes), host(w.absmax_q), host(w.absmax_scale)
        for gi in _sample_groups(ng, 48, i):
            e0, e1 = gi * 16384, min(n, (gi + 1) * 16384)
            seg = syn.torch_bf16_to_bits(flat[e0:e1])
            codes, q8, s2 = oracle.quantize_nf4_dq(seg, "bf16")
            assert np.array_equal(gc[e0 // 2:e1 // 2], codes), (name, gi)
            assert np.array_equal(gq[e0 // 64:e1 // 64], q8), (name, gi)
            assert gs[gi].view(np.uint32) == s2[0].view(np.uint32), (name, gi)
        del W, w
    torch.cuda.empty_cache()


def test_bulk_65b_student_t_resident_and_roundtrip():
    """277 heavy-tailed 8192x28672 tensors (65e9 weights) quantized on one GPU,
    all NF4 buffers kept resident; tensors 0, 138, 276 bit-exact against the
    oracle; every tensor's dequant round trip within the per-element bound."""
    cfg = syn.BULK_65B
    shape, T = cfg["tensor"], cfg["n_tensors"]
    lv, _ = oracle.nf4_codebook()
    halfgap = float(np.max(np.diff(lv.astype(np.float64))) / 2)
    resident = []
    checked = {0, 138, 276}
    futures = {}
    for t in range(T):
        W = syn.torch_student_t_outliers_bf16(shape, syn.seed_of(5, t), DEV)
        w = q.qlora_quantize_nf4_dq(W)
        if t in checked:
            torch.cuda.synchronize()
            Wb = syn.torch_bf16_to_bits(W)
            futures[t] = (POOL.submit(oracle.quantize_nf4_dq, Wb, "bf16"),
                          host(w.codes), host(w.absmax_q), host(w.absmax_scale))
        resident.append(w)
        if t % 20 == 0:
            say("bulk quantize", t, "of", T)
        del W
    torch.cuda.synchronize()
    total = sum(w.nbytes() for w in resident)
    n_params = T * shape[0] * shape[1]
    assert total * 8 / n_params == 4.126953125
    say("resident NF4 bytes", total)
    # round trip: |w - w_hat| <= c1 * halfgap + |c1 - c1_hat| + small, per element
    for t in range(T):
        W = syn.torch_student_t_outliers_bf16(shape, syn.seed_of(5, t), DEV).float().view(-1, 64)
        deq = q.qlora_dequant_bf16(resident[t]).float().view(-1, 64)
        c1 = W.abs().amax(dim=1, keepdim=True)
        qa = resident[t].absmax_q.float().view(-1, 1)
        s2 = resident[t].absmax_scale.repeat_interleave(256)[: qa.shape[0]].view(-1, 1)
        c1h = qa * s2
        bound = c1 * (halfgap + 2.0 ** -22) + (c1 - c1h).abs() + c1h.abs() * 2.0 ** -7
        assert bool(((W - deq).abs() <= bound).all()), f"round-trip bound, tensor {t}"
        del W, deq
    for t, (fut, gc, gq, gs) in futures.items():
        codes, q8, s2 = fut.result()
        assert np.array_equal(gc, codes), f"bulk tensor {t} codes"
        assert np.array_equal(gq, q8), f"bulk tensor {t} absmax codes"
        assert np.array_equal(gs.view(np.uint32), s2.view(np.uint32)), f"bulk tensor {t} scales"
    del resident
    torch.cuda.empty_cache()


def test_quantize_deterministic():
    W = syn.torch_normal_bf16((512, 4096), 0.02, 7, DEV)
    a, b = quantize_gpu(W), quantize_gpu(W)
    assert torch.equal(a.codes, b.codes) and torch.equal(a.absmax_q, b.absmax_q)


# ------------------------------------------------------------------ linear layer helpers
class Problem:
    """A seeded layer problem with both sides' inputs and the oracle's W_hat."""

    def __init__(self, N, K, r, alpha, w_std=0.02, seed=0, w_dtype="bf16", zero_w=False, fmt=0):
        self.N, self.K, self.r, self.alpha = N, K, r, alpha
        if zero_w:
            Wb = np.zeros((N, K), np.uint16)
        else:
            Wb = syn.normal_bf16((N, K), w_std, seed) if w_dtype == "bf16" else None
        if w_dtype == "f32":
            Wf = syn.normal_f32((N, K), w_std, seed)
            self.w = quantize_gpu(torch.from_numpy(Wf).to(DEV), fmt)
            codes, q8, s2 = oracle.quantize_nf4_dq(Wf, "f32", fmt)
        else:
            self.w = quantize_gpu(dev_bf16(Wb), fmt)
            codes, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16", fmt)
        assert_nf4_equal(self.w, codes, q8, s2, "problem weight")
        self.What = oracle.dequant_dq(codes, q8, s2, fmt)[1].reshape(N, K)
        self.A = syn.normal_bf16((K, r), 1.0 / np.sqrt(K), seed + 1)
        self.B = syn.normal_bf16((r, N), 0.01, seed + 2)
        self.At, self.Bt = dev_bf16(self.A), dev_bf16(self.B)


def run_fwd(P, x, **kw):
    y = q.qlora_linear_fwd(P.w, dev_bf16(x), P.At, P.Bt, P.alpha, **kw)
    torch.cuda.synchronize()
    return y


# ------------------------------------------------------------------ forward
@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("name", ["q", "up"])
def test_fwd_decode_llama7b(M, name):
    cfg = syn.LLAMA7B_DECODE
    N, K = cfg["weights"][name]
    say("fwd decode", name, M)
    P = Problem(N, K, cfg["r"], cfg["alpha"], seed=syn.seed_of(2, 10 + (name == "up")))
    x = syn.normal_bf16((M, K), 1.0, syn.seed_of(2, 20 + M))
    y = host(run_fwd(P, x))
    yo, _ = oracle.linear_fwd(x, P.What, P.A, P.B, P.r, P.alpha)
    tol_check(y, yo, f"y decode {name} M={M}")


@pytest.mark.parametrize("M,N,K,r", [(17, 320, 640, 16), (300, 100, 192, 32), (256, 512, 1024, 64),
                                     (33, 1024, 128, 16), (8, 72, 64, 16),
                                     # large-M path: ragged tile rows and columns, step tails
                                     (600, 520, 192, 16), (512, 256, 64, 32), (700, 300, 1024, 64),
                                     # single-pass down projection with two rank tiles
                                     # (M >= 2048, r = 32), ragged last 16-row tile
                                     (2056, 544, 640, 32),
                                     # fused large-M kernel: one-block rows (K = 64), pair
                                     # counts off the four-pair unroll (5, 7), weight rows
                                     # that leave waves or whole 32-row halves empty
                                     (1024, 1000, 64, 16), (520, 100, 320, 16),
                                     (513, 40, 448, 32), (777, 289, 192, 48),
                                     # tiled down projection: 128-row tiles, 512-wide
                                     # slices with a ragged last one, r = 64 and 96
                                     (1024, 520, 1088, 64), (1100, 200, 320, 96),
                                     # few output tiles: the dense stage splits the
                                     # reduction (eight splits of 16 steps)
                                     (600, 300, 4096, 16), (520, 1024, 8192, 64),
                                     # streaming down projection: 64-wide chunks, an odd
                                     # count (65), ragged 128-row blocks, r = 32 and 96
                                     (600, 520, 4160, 32), (1030, 300, 4096, 96),
                                     # 16 < M < 512 with few tiles: the reduction over K
                                     # split into ranges of blocks (22 ranges, the last
                                     # of two blocks; 8 ranges)
                                     (64, 1000, 4160, 16), (130, 2048, 1024, 32),
                                     # the tiled down projection (M >= 1024, r >= 64,
                                     # 2048 <= K < 4096: 128 workgroups)
                                     (4096, 256, 2048, 64)])
def test_fwd_full_small(M, N, K, r):
    say("fwd small", M, N, K, r)
    P = Problem(N, K, r, 32.0, seed=M + N + K)
    x = syn.normal_bf16((M, K), 1.0, 7 + M)
    yo, _ = oracle.linear_fwd(x, P.What, P.A, P.B, r, 32.0)
    # from 512 rows on both routes: one bf16 copy of the weight in the
    # workspace (fast) and the fused in-register dequantization (lean)
    for lean in ((False, True) if M >= 512 else (False,)):
        y = host(run_fwd(P, x, lean=lean))
        tol_check(y, yo, f"y {M}x{N}x{K} lean={lean}")
        # bf16 output is the RNE rounding of the fp32 output of the same computation
        yb = run_fwd(P, x, y_dtype=torch.bfloat16, lean=lean)
        assert torch.equal(yb, torch.from_numpy(y).to(torch.bfloat16).to(DEV))


def test_fwd_linear_1024_f32_weight():
    cfg = syn.LINEAR_1024
    N, K = cfg["weights"]["w"]
    P = Problem(N, K, cfg["r"], cfg["alpha"], seed=syn.seed_of(1, 0), w_dtype="f32")
    x = syn.normal_bf16((cfg["M"], K), 1.0, syn.seed_of(1, 3))
    y = host(run_fwd(P, x))
    yo, _ = oracle.linear_fwd(x, P.What, P.A, P.B, P.r, P.alpha)
    tol_check(y, yo, "y 1024")


@pytest.mark.parametrize("name", ["q", "up"])
def test_fwd_train_llama7b_sampled_rows(name):
    cfg = syn.LLAMA7B_TRAIN
    N, K = cfg["weights"][name]
    M = cfg["M"]
    say("fwd train", name)
    P = Problem(N, K, cfg["r"], cfg["alpha"], seed=syn.seed_of(3, 10 + (name == "up")))
    x = syn.normal_bf16((M, K), 1.0, syn.seed_of(3, 20))
    u = torch.empty((M, P.r), dtype=torch.float32, device=DEV)
    y = run_fwd(P, x, u_out=u)
    rows = np.array(sorted(set(np.random.default_rng(1).choice(M, 24, replace=False).tolist())
                           | {0, 255, 256, M - 1}))
    yo, uo = oracle.linear_fwd(x[rows], P.What, P.A, P.B, P.r, P.alpha)
    tol_check(host(y)[rows], yo, f"y train {name}")
    tol_check(host(u)[rows], uo, f"u train {name}")
    yl = run_fwd(P, x, lean=True)
    tol_check(host(yl)[rows], yo, f"y train {name} lean")


def test_fwd_one_hot_rows_exact_gemm_and_gemv():
    """x rows one-hot, B = 0: y rows equal dequantized weight columns exactly,
    which pins the in-kernel dequantization to the standalone one."""
    N, K, r = 512, 1024, 16
    P = Problem(N, K, r, 32.0, seed=5)
    P.Bt = torch.zeros_like(P.Bt)
    for M, lean in ((2, False), (4, False), (16, False), (64, False), (600, False), (600, True)):
        ks = np.random.default_rng(M).choice(K, M, replace=False)
        x = np.zeros((M, K), np.uint16)
        x[np.arange(M), ks] = 0x3F80
        y = host(run_fwd(P, x, lean=lean))
        Wf = oracle.bf16_to_f32(P.What)
        assert np.array_equal(y, Wf[:, ks].T + 0.0), f"one-hot M={M} lean={lean}"


def test_fwd_lora_only_isolated():
    """All codes at the zero level: y is the adapter term alone."""
    N, K, r = 384, 512, 16
    P = Problem(N, K, r, 32.0, seed=9, zero_w=True)
    assert int(host(P.w.codes).min()) == 0x77 == int(host(P.w.codes).max())
    for M in (5, 100):
        x = syn.normal_bf16((M, K), 1.0, 70 + M)
        y = host(run_fwd(P, x))
        yo, _ = oracle.linear_fwd(x, P.What, P.A, P.B, r, 32.0)
        tol_check(y, yo, f"lora-only M={M}")


@pytest.mark.parametrize("M", [300, 600])
def test_fwd_deterministic(M):
    P = Problem(1024, 1024, 16, 32.0, seed=3)
    x = syn.normal_bf16((M, 1024), 1.0, 4)
    a, b = run_fwd(P, x), run_fwd(P, x)
    assert torch.equal(a, b)


# hipStreamPerThread, a second stream beside torch's current one.
PER_THREAD_STREAM = types.SimpleNamespace(cuda_stream=2)


def run_fwd_other_stream(P, x, **kw):
    torch.cuda.synchronize()
    y = q.qlora_linear_fwd(P.w, dev_bf16(x), P.At, P.Bt, P.alpha, stream=PER_THREAD_STREAM, **kw)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M,N,K,r", [(1, 72, 64, 16), (3, 330, 192, 32), (16, 100, 320, 16),
                                     (7, 1000, 1600, 64), (2, 40, 4096, 144),
                                     # four waves per tile (>= 512 tiles), ragged rows
                                     (16, 8200, 512, 16), (3, 8200, 256, 80),
                                     # one-round-trip kernel (M <= 4, K % 256 == 0,
                                     # K <= 4096, r <= 32): eight waves per tile
                                     # (under 1024 tiles) with a ragged last tile
                                     # and lanes past the row end, x slices for two
                                     # or for four tokens; four waves per tile
                                     # (>= 1024 tiles)
                                     (1, 100, 256, 16), (2, 300, 4096, 32),
                                     (2, 8200, 768, 32), (1, 8192, 4096, 16),
                                     (3, 100, 256, 16), (4, 520, 4096, 32),
                                     (1, 16400, 256, 16), (4, 16400, 512, 32),
                                     (3, 16392, 256, 16)])
def test_fwd_decode_ragged(M, N, K, r):
    """Decode (M <= 16): ragged rows, chunks and adapter column groups against
    the oracle; a call on another stream gives the same bits."""
    say("fwd decode ragged", M, N, K, r)
    P = Problem(N, K, r, 24.0, seed=N + K + r)
    x = syn.normal_bf16((M, K), 1.0, 11 + M)
    u1 = torch.empty((M, r), dtype=torch.float32, device=DEV)
    y1 = run_fwd(P, x, u_out=u1)
    yo, uo = oracle.linear_fwd(x, P.What, P.A, P.B, r, 24.0)
    tol_check(host(y1), yo, f"y decode {M}x{N}x{K} r{r}")
    tol_check(host(u1), uo, f"u decode {M}x{N}x{K} r{r}")
    u2 = torch.empty_like(u1)
    y2 = run_fwd_other_stream(P, x, u_out=u2)
    assert torch.equal(y1, y2), "y differs between streams"
    assert torch.equal(u1, u2), "u differs between streams"
    yb = run_fwd(P, x, y_dtype=torch.bfloat16)
    assert torch.equal(yb, y1.to(torch.bfloat16))


def test_fwd_decode_repeat_streams_and_graph():
    """Back-to-back decode calls on one stream, calls on two streams and the
    replays of a captured call (eager work in between) each match a separate
    call on another stream for their input, bit for bit."""
    N, K, r, M, alpha = 4100, 1024, 32, 4, 32.0
    P = Problem(N, K, r, alpha, seed=21)
    xs = [syn.normal_bf16((M, K), 1.0, 300 + t) for t in range(3)]
    ref = [run_fwd_other_stream(P, x) for x in xs]
    xd = [dev_bf16(x) for x in xs]
    torch.cuda.synchronize()
    ys = [q.qlora_linear_fwd(P.w, xv, P.At, P.Bt, alpha) for xv in xd]  # no sync in between
    torch.cuda.synchronize()
    for t in range(3):
        assert torch.equal(ys[t], ref[t]), f"back-to-back call {t}"
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        ya = q.qlora_linear_fwd(P.w, xd[0], P.At, P.Bt, alpha)
    with torch.cuda.stream(s2):
        yb = q.qlora_linear_fwd(P.w, xd[1], P.At, P.Bt, alpha)
    torch.cuda.synchronize()
    assert torch.equal(ya, ref[0]) and torch.equal(yb, ref[1]), "two streams"
    xin = xd[0].clone()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        yg = q.qlora_linear_fwd(P.w, xin, P.At, P.Bt, alpha)
    for rep in range(6):
        t = rep % 3
        xin.copy_(xd[t])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, ref[t]), f"graph replay {rep}"
        ye = q.qlora_linear_fwd(P.w, xd[(t + 1) % 3], P.At, P.Bt, alpha)
        torch.cuda.synchronize()
        assert torch.equal(ye, ref[(t + 1) % 3]), f"eager call after replay {rep}"


@pytest.mark.parametrize("M,N,K,r,pad", [(300, 520, 96, 16, 0), (513, 256, 64, 32, 24),
                                         (256, 256, 32, 16, 0), (40, 1030, 320, 64, 8)])
def test_gemm_bf16_nt_dense_stage(M, N, K, r, pad):
    """The dense stage on its own: y = a b^T + e [f|f]^T against the fp64
    product of the same bf16 inputs; a given with a row stride K + pad."""
    say("gemm nt", M, N, K, r, pad)
    a_full = syn.normal_bf16((M, K + pad), 1.0, 50 + M)
    b = syn.normal_bf16((N, K), 0.05, 51 + N)
    e = syn.normal_bf16((M, 2 * r), 1.0, 52 + r)
    f = syn.normal_bf16((N, r), 0.1, 53 + K)
    at, bt, et, ft = dev_bf16(a_full), dev_bf16(b), dev_bf16(e), dev_bf16(f)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    L = q._lib.load()
    P_ = ctypes.c_void_p
    st = L.qlora_gemm_bf16_nt(P_(at.data_ptr()), K + pad, P_(bt.data_ptr()), K, q.LAYOUT_ROWS,
                              P_(et.data_ptr()), P_(ft.data_ptr()), M, N, K, r, P_(y.data_ptr()),
                              0, P_(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    f64 = lambda v: oracle.bf16_to_f32(v).astype(np.float64)
    ref = f64(a_full[:, :K]) @ f64(b).T + f64(e) @ np.concatenate([f64(f), f64(f)], 1).T
    tol_check(host(y), ref, f"gemm nt {M}x{N}x{K}")
    if pad == 0:
        yb = q.qlora_gemm_bf16_nt(at, bt, et, ft, y_dtype=torch.bfloat16)
        assert torch.equal(yb, y.to(torch.bfloat16))
    # b in the K-slab layout [K/32, N, 32]: the same tiles reach the MFMAs,
    # so y is the same bit for bit
    b_slab = bt.view(N, K // 32, 32).transpose(0, 1).contiguous()
    ys = torch.empty_like(y)
    st = L.qlora_gemm_bf16_nt(P_(at.data_ptr()), K + pad, P_(b_slab.data_ptr()), 0,
                              q.LAYOUT_KSLAB32, P_(et.data_ptr()), P_(ft.data_ptr()), M, N, K, r,
                              P_(ys.data_ptr()), 0, P_(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(ys, y), "K-slab b"


@pytest.mark.parametrize("N,K", [(257, 640), (64, 64), (11008, 4096)])
def test_dequant_kslab_layout_bit_exact(N, K):
    """The K-slab layout [K/32, N, 32] holds exactly the oracle's w_hat."""
    say("dequant kslab", N, K)
    Wb = syn.normal_bf16((N, K), 0.02, 70 + N)
    w = quantize_gpu(dev_bf16(Wb))
    got = syn.torch_bf16_to_bits(q.qlora_dequant_bf16(w, layout=q.LAYOUT_KSLAB32))
    codes, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16")
    want = oracle.dequant_dq(codes, q8, s2)[1].reshape(N, K // 32, 32).transpose(1, 0, 2)
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ backward
def run_bwd(P, x, dY, **kw):
    out = q.qlora_linear_bwd(P.w, None if x is None else dev_bf16(x), dev_bf16(dY), P.At, P.Bt,
                             P.alpha, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("M,N,K,r", [(16, 1024, 1024, 16), (300, 100, 192, 32), (64, 512, 640, 64),
                                     (8, 72, 64, 16), (257, 256, 256, 16),
                                     # large-M path (reduction over N = 544, 320)
                                     (600, 544, 192, 16), (520, 320, 640, 32),
                                     # single-pass down projections (v over N, the
                                     # recomputed u over K) with r = 32, M >= 2048,
                                     # and r = 64 (two 32-wide rank blocks)
                                     (2056, 544, 640, 32), (2056, 544, 640, 64),
                                     # tiled down projections (128-row tiles, 512-wide
                                     # slices, two rank chunks at r = 96), ragged M
                                     (1100, 200, 1088, 64), (1030, 520, 320, 96),
                                     # dX from 512 rows with N % 32 != 0: the tile
                                     # kernel (N % 8 == 0) and the general one
                                     (600, 1000, 192, 16), (520, 1100, 320, 32),
                                     (600, 100, 128, 16),
                                     # few dX tiles: the reduction over N is split
                                     (600, 4096, 512, 16),
                                     # streaming down projections: v over N = 4104 (a
                                     # last chunk of 8), u over K = 4160, r = 32 and 96
                                     (600, 4104, 320, 32), (1030, 4096, 4160, 96),
                                     # small M: dX's reduction over N split into
                                     # ranges (11 with a last step of 8 rows and a
                                     # 64-column last tile; 32)
                                     (3, 2056, 320, 16), (16, 4096, 1024, 64)])
def test_bwd_full_small(M, N, K, r):
    say("bwd small", M, N, K, r)
    P = Problem(N, K, r, 24.0, seed=M + 2 * N + K)
    x = syn.normal_bf16((M, K), 1.0, 3 + M)
    dY = syn.normal_bf16((M, N), 1.0, 4 + M)
    go = oracle.linear_bwd(x, dY, P.What, P.A, P.B, r, 24.0)
    # from 512 rows on both routes: dX through one transposed bf16 copy of the
    # weight (fast) and through the in-register kernel (lean)
    for lean in ((False, True) if M >= 512 else (False,)):
        dX, dA, dB = run_bwd(P, x, dY, lean=lean)
        tol_check(host(dX), go["dX"], f"dX lean={lean}")
        tol_check(host(dA), go["dA"], f"dA lean={lean}")
        tol_check(host(dB), go["dB"], f"dB lean={lean}")
        # bf16 outputs are the RNE of the fp32 ones
        dXb, dAb, dBb = run_bwd(P, x, dY, dx_dtype=torch.bfloat16, grad_dtype=torch.bfloat16,
                                lean=lean)
        assert torch.equal(dXb, dX.to(torch.bfloat16))
        assert torch.equal(dAb, dA.to(torch.bfloat16)) and torch.equal(dBb, dB.to(torch.bfloat16))


@pytest.mark.parametrize("M,N,K,r", [(5, 520, 1024, 32), (16, 300, 4096, 16),
                                     (1100, 200, 1088, 64), (2056, 544, 640, 64)])
def test_bwd_decode_recomputed_u_matches_saved(M, N, K, r):
    """The backward recomputes u with the forward's down projection and slice
    sum (at decode sizes, through the tiled kernel, and through the
    single-pass kernel, whose launch for v also splits a saved u): the same
    bits as the u the forward returns, so dA and dB agree exactly with
    u_saved given or not."""
    P = Problem(N, K, r, 24.0, seed=M + N)
    x = syn.normal_bf16((M, K), 1.0, 40 + M)
    dY = syn.normal_bf16((M, N), 1.0, 41 + M)
    u = torch.empty((M, r), dtype=torch.float32, device=DEV)
    run_fwd(P, x, u_out=u)
    _, dA1, dB1 = run_bwd(P, x, dY, u_saved=u, want_dx=False)
    _, dA2, dB2 = run_bwd(P, x, dY, want_dx=False)
    assert torch.equal(dA1, dA2) and torch.equal(dB1, dB2)
    go = oracle.linear_bwd(x, dY, P.What, P.A, P.B, r, 24.0, ("dA", "dB"))
    tol_check(host(dB2), go["dB"], "dB decode")


def _bwd_abi(P, xd, dYd, dA, dB):
    """qlora_linear_bwd through the C ABI with either adapter gradient
    optional (NULL), no dX; fp32 gradients."""
    M, r = dYd.shape[0], P.At.shape[1]
    ws = torch.empty(q.qlora_workspace_bytes(1, M, P.w.N, P.w.K, r), dtype=torch.uint8, device=DEV)
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = q._lib.load().qlora_linear_bwd(
        P.w.desc(), ptr(xd), ptr(dYd), M, ptr(P.At), ptr(P.Bt), r, float(P.alpha), None, None, 0,
        ptr(dA), ptr(dB), 0, ptr(ws), ws.numel(), None)
    torch.cuda.synchronize()
    assert st == 0, q.qlora_strerror(st)


@pytest.mark.parametrize("M,N,K,r", [(4096, 1100, 640, 16), (300, 100, 192, 32), (16, 520, 1024, 16)])
def test_bwd_single_adapter_gradient_matches_both(M, N, K, r):
    """dA alone and dB alone (the other NULL) run the reduction launches with
    one job instead of two; each equals the same gradient of the call that
    asks for both, bit for bit."""
    say("bwd single gradient", M, N, K, r)
    P = Problem(N, K, r, 32.0, seed=M + 3 * N)
    x = syn.normal_bf16((M, K), 1.0, 50 + M)
    dY = syn.normal_bf16((M, N), 1.0, 51 + M)
    xd, dYd = dev_bf16(x), dev_bf16(dY)
    _, dA, dB = run_bwd(P, x, dY, want_dx=False)
    dA1 = torch.full_like(dA, float("nan"))
    dB1 = torch.full_like(dB, float("nan"))
    _bwd_abi(P, xd, dYd, dA1, None)
    _bwd_abi(P, xd, dYd, None, dB1)
    assert torch.equal(dA1, dA) and torch.equal(dB1, dB)


def test_bwd_direct_gradients_single_matches_both():
    """Shapes whose adapter gradients take the direct reduction (one launch
    per call, no slices): dA alone and dB alone equal the gradients of the
    call that asks for both, bit for bit, and a 64-row tail of M pads with
    zeros. The weight is quantized on the GPU only: both sides are this
    library."""
    for M, N, K, r in [(520, 8192, 8192, 16), (300, 24576, 8192, 64)]:
        say("direct gradients", M, N, K, r)
        W = syn.torch_normal_bf16((N, K), 0.02, syn.seed_of(9, N), DEV)
        w = quantize_gpu(W)
        del W
        A = dev_bf16(syn.normal_bf16((K, r), 1.0 / np.sqrt(K), 61))
        B = dev_bf16(syn.normal_bf16((r, N), 0.01, 62))
        xd = dev_bf16(syn.normal_bf16((M, K), 1.0, 63))
        dYd = dev_bf16(syn.normal_bf16((M, N), 1.0, 64))
        P = types.SimpleNamespace(w=w, At=A, Bt=B, alpha=16.0, N=N, K=K, r=r)
        _, dA, dB = q.qlora_linear_bwd(w, xd, dYd, A, B, 16.0, want_dx=False)
        torch.cuda.synchronize()
        dA1 = torch.full_like(dA, float("nan"))
        dB1 = torch.full_like(dB, float("nan"))
        _bwd_abi(P, xd, dYd, dA1, None)
        _bwd_abi(P, xd, dYd, None, dB1)
        assert torch.equal(dA1, dA) and torch.equal(dB1, dB), (M, N, K, r)
        del w, xd, dYd
        torch.cuda.empty_cache()


def test_bwd_linear_1024_f32_weight():
    cfg = syn.LINEAR_1024
    N, K = cfg["weights"]["w"]
    P = Problem(N, K, cfg["r"], cfg["alpha"], seed=syn.seed_of(1, 0), w_dtype="f32")
    x = syn.normal_bf16((cfg["M"], K), 1.0, syn.seed_of(1, 3))
    dY = syn.normal_bf16((cfg["M"], N), 1.0, syn.seed_of(1, 4))
    u = torch.empty((cfg["M"], P.r), dtype=torch.float32, device=DEV)
    run_fwd(P, x, u_out=u)
    dX, dA, dB = run_bwd(P, x, dY, u_saved=u)
    go = oracle.linear_bwd(x, dY, P.What, P.A, P.B, P.r, P.alpha)
    for got, k in ((dX, "dX"), (dA, "dA"), (dB, "dB")):
        tol_check(host(got), go[k], k + " 1024")
    # saved u and recomputed u give the same dB bits
    _, _, dB2 = run_bwd(P, x, dY)
    assert torch.equal(dB, dB2)


@pytest.mark.parametrize("name", ["q", "up"])
def test_bwd_train_llama7b(name):
    cfg = syn.LLAMA7B_TRAIN
    N, K = cfg["weights"][name]
    M = cfg["M"]
    say("bwd train", name)
    P = Problem(N, K, cfg["r"], cfg["alpha"], seed=syn.seed_of(3, 10 + (name == "up")))
    x = syn.normal_bf16((M, K), 1.0, syn.seed_of(3, 20))
    dY = syn.normal_bf16((M, N), 1.0, syn.seed_of(3, 30 + (name == "up")))
    dX, dA, dB = run_bwd(P, x, dY)
    rows = np.array(sorted(set(np.random.default_rng(2).choice(M, 24, replace=False).tolist())
                           | {0, 255, 256, M - 1}))
    f_dx = POOL.submit(oracle.linear_bwd, x[rows], dY[rows], P.What, P.A, P.B, P.r, P.alpha,
                       ("dX",))
    f_g = POOL.submit(oracle.linear_bwd, x, dY, P.What, P.A, P.B, P.r, P.alpha, ("dA", "dB"))
    tol_check(host(dX)[rows], f_dx.result()["dX"], f"dX train {name}")
    g = f_g.result()
    tol_check(host(dA), g["dA"], f"dA train {name}")
    tol_check(host(dB), g["dB"], f"dB train {name}")


@pytest.mark.parametrize("M,N,K", [(40, 320, 512), (600, 640, 512), (16, 1024, 512),
                                   # from 512 rows, N % 32 == 0: the transposed copy's
                                   # last column tile is ragged (K % 256 = 64)
                                   (512, 544, 320), (520, 672, 4160)])
def test_bwd_one_hot_dy_rows_exact(M, N, K):
    r = 16
    P = Problem(N, K, r, 32.0, seed=11)
    P.Bt = torch.zeros_like(P.Bt)
    ns = np.random.default_rng(4).choice(N, M, replace=False)
    dY = np.zeros((M, N), np.uint16)
    dY[np.arange(M), ns] = 0x3F80
    Wf = oracle.bf16_to_f32(P.What)
    for lean in ((False, True) if M >= 512 else (False,)):
        dX, _, _ = run_bwd(P, None, dY, want_grads=False, lean=lean)
        assert np.array_equal(host(dX), Wf[ns] + 0.0), f"lean={lean}"


def test_bwd_empty_batch_gives_zero_grads():
    P = Problem(128, 256, 16, 32.0, seed=12)
    x = np.zeros((0, 256), np.uint16)
    dY = np.zeros((0, 128), np.uint16)
    dX, dA, dB = run_bwd(P, x, dY)
    assert dX.shape == (0, 256)
    assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) == 0


def test_layer_70b_fwd_bwd_sampled():
    """All 7 projections of the 70B-shaped layer at M = 2048, r = 64, alpha = 16:
    y and dX on 12 sampled rows, dA and dB in full."""
    cfg = syn.LAYER_70B
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    rows = np.array([0, 1, 255, 256, 511, 1000, 1023, 1024, 1500, 2046, 2047, 777])
    x_shared = syn.normal_bf16((M, 8192), 1.0, syn.seed_of(4, 100))
    jobs = []
    for i, (name, (N, K)) in enumerate(cfg["weights"].items()):
        say("70b layer", name, N, K)
        Wd = syn.torch_normal_bf16((N, K), cfg["w_std"], syn.seed_of(4, i), DEV)
        w = quantize_gpu(Wd)
        Wb = syn.torch_bf16_to_bits(Wd)
        del Wd
        x = x_shared if name not in ("o", "down") else syn.normal_bf16((M, K), 1.0,
                                                                       syn.seed_of(4, 110 + i))
        A = syn.normal_bf16((K, r), 1.0 / np.sqrt(K), syn.seed_of(4, 20 + i))
        B = syn.normal_bf16((r, N), 0.01, syn.seed_of(4, 30 + i))
        dY = syn.normal_bf16((M, N), 1.0, syn.seed_of(4, 40 + i))
        xt, At, Bt, dYt = dev_bf16(x), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
        u = torch.empty((M, r), dtype=torch.float32, device=DEV)
        y = q.qlora_linear_fwd(w, xt, At, Bt, alpha, u_out=u)
        dX, dA, dB = q.qlora_linear_bwd(w, xt, dYt, At, Bt, alpha, u_saved=u)
        torch.cuda.synchronize()
        got = (host(y)[rows], host(dX)[rows], host(dA), host(dB))
        del w, y, dX, dA, dB, xt, dYt, u

        def oracle_job(x=x, Wb=Wb, A=A, B=B, dY=dY):
            codes, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16")
            What = oracle.dequant_dq(codes, q8, s2)[1].reshape(Wb.shape)
            yo, _ = oracle.linear_fwd(x[rows], What, A, B, r, alpha)
            gx = oracle.linear_bwd(x[rows], dY[rows], What, A, B, r, alpha, ("dX",))
            gab = oracle.linear_bwd(x, dY, What, A, B, r, alpha, ("dA", "dB"))
            return yo, gx["dX"], gab["dA"], gab["dB"]

        jobs.append((name, got, POOL.submit(oracle_job)))
        torch.cuda.empty_cache()
    for name, got, fut in jobs:
        ref = fut.result()
        for g, rr, k in zip(got, ref, ("y", "dX", "dA", "dB")):
            tol_check(g, rr, f"70b {name} {k}")
        say("70b layer ok", name)


# ------------------------------------------------------- beyond 2^31 bytes
def test_fwd_bwd_weight_past_2gib_of_bf16():
    """A weight whose bf16 copy is past 2^31 bytes (16448 x 65536, 1.08G
    weights) at M = 512: the forward takes the fused route (the dense
    stage's 32-bit offsets cannot hold the copy) and the backward's dX the
    tile kernel. Sampled rows of y and dX against the oracle, which quantizes
    the same bf16 weight itself."""
    N, K, M, r = 16448, 65536, 512, 16
    say("weight past 2 GiB", N, K)
    assert 2 * N * K >= 2 ** 31
    Wb = syn.normal_bf16((N, K), 0.02, 90)
    w = quantize_gpu(dev_bf16(Wb))
    codes, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16")
    del Wb
    assert_nf4_equal(w, codes, q8, s2, "weight past 2 GiB")
    What = oracle.dequant_dq(codes, q8, s2)[1].reshape(N, K)
    del codes, q8, s2
    A = syn.normal_bf16((K, r), 1.0 / np.sqrt(K), 91)
    B = syn.normal_bf16((r, N), 0.01, 92)
    x = syn.normal_bf16((M, K), 1.0, 93)
    dY = syn.normal_bf16((M, N), 1.0, 94)
    At, Bt = dev_bf16(A), dev_bf16(B)
    assert q.qlora_workspace_bytes(0, M, N, K, r) == q.qlora_workspace_bytes(3, M, N, K, r)
    y = q.qlora_linear_fwd(w, dev_bf16(x), At, Bt, 32.0)
    dX, _, _ = q.qlora_linear_bwd(w, None, dev_bf16(dY), At, Bt, 32.0, want_grads=False)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 300, M - 1])
    yo, _ = oracle.linear_fwd(x[rows], What, A, B, r, 32.0)
    tol_check(host(y)[rows], yo, "y past 2 GiB")
    go = oracle.linear_bwd(x[rows], dY[rows], What, A, B, r, 32.0, ("dX",))
    tol_check(host(dX)[rows], go["dX"], "dX past 2 GiB")


# ------------------------------------------------------------ descriptor
@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_quantize_records_the_setup_and_calls_check_it(fmt):
    """[P4] "Operational coupling": quantizing records the format version and
    the setup id in the weight's descriptor; a descriptor relabelled to
    another second-level format, or carrying another setup id, is refused by
    every reading call before anything is launched."""
    N, K, r = 96, 256, 16
    say("descriptor", fmt)
    w = quantize_gpu(dev_bf16(syn.normal_bf16((N, K), 0.02, 80 + fmt)), fmt)
    assert w.format_version == 1 and w.setup_id == q.qlora_setup_id(fmt)
    assert q.qlora_nf4_check(w) == 0
    x = dev_bf16(syn.normal_bf16((32, K), 1.0, 83))
    A = dev_bf16(syn.normal_bf16((K, r), 0.05, 84))
    B = dev_bf16(syn.normal_bf16((r, N), 0.01, 85))
    y0 = q.qlora_linear_fwd(w, x, A, B, 32.0)
    torch.cuda.synchronize()
    relabelled = q.NF4Weight(w.codes, w.absmax_q, w.absmax_scale, N, K, (fmt + 1) % 3,
                             w.format_version, w.setup_id)
    foreign = q.NF4Weight(w.codes, w.absmax_q, w.absmax_scale, N, K, fmt, w.format_version,
                          w.setup_id ^ 0x5A5A)
    for bad in (relabelled, foreign):
        assert q.qlora_nf4_check(bad) == 9
        y = torch.full((32, N), 7.0, device=DEV)
        with pytest.raises(RuntimeError, match="setup"):
            q.qlora_linear_fwd(bad, x, A, B, 32.0, y=y)
        with pytest.raises(RuntimeError, match="setup"):
            q.qlora_dequant_bf16(bad)
        with pytest.raises(RuntimeError, match="setup"):
            q.qlora_linear_bwd(bad, x, dev_bf16(syn.normal_bf16((32, N), 1.0, 86)), A, B, 32.0)
        torch.cuda.synchronize()
        assert torch.all(y == 7.0)  # nothing was launched
    assert torch.equal(q.qlora_linear_fwd(w, x, A, B, 32.0), y0)


# ------------------------------------------------------------------- merge
@pytest.mark.parametrize("N,K,r,base", [(1024, 1024, 16, "nf4"), (1024, 1024, 16, "bf16"),
                                        (257, 640, 32, "nf4"), (72, 64, 64, "bf16"),
                                        (11008, 4096, 16, "nf4")])
def test_merge_and_requantize_bit_exact(N, K, r, base):
    """merged = base + s (A B)^T bit for bit against the oracle, then the
    requantized codes, 8-bit scale codes and second-level scales bit for bit."""
    say("merge", N, K, r, base)
    Wb = syn.normal_bf16((N, K), 0.02, 60 + r)
    A = syn.normal_bf16((K, r), 1.0 / np.sqrt(K), 61 + r)
    B = syn.normal_bf16((r, N), 0.01, 62 + r)
    At, Bt = dev_bf16(A), dev_bf16(B)
    if base == "nf4":
        w = quantize_gpu(dev_bf16(Wb))
        codes, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16")
        merged = q.qlora_merge_lora(At, Bt, 32.0, w=w)
        ref = oracle.merge_lora(A, B, r, 32.0, nf4=(codes, q8, s2, N, K))
    else:
        merged = q.qlora_merge_lora(At, Bt, 32.0, W=dev_bf16(Wb))
        ref = oracle.merge_lora(A, B, r, 32.0, W=Wb)
    torch.cuda.synchronize()
    got = host(merged)
    assert got.dtype == np.float32
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "merged weight bits"
    wq = q.qlora_quantize_nf4_dq(merged)
    assert_nf4_equal(wq, *oracle.quantize_nf4_dq(ref, "f32"), f"requantized {base}")


@pytest.mark.parametrize("base", ["nf4", "bf16"])
def test_merge_subnormal_products_bit_exact(base):
    """Products of the adapter terms below the normal range, where rounding
    each product before the add differs from a fused multiply-add: A and B
    ~ N(0,1) x 2^-72, zero base, alpha = r, so merged = the adapter sum
    itself. Bit for bit against the oracle, plus the closed-form rank-2 case
    (products 2^-149 and 2^-150 sum to exactly 2^-149)."""
    N, K, r = 136, 192, 16
    say("merge subnormal products", base)
    rng = np.random.default_rng(64)
    A = syn.to_bf16_bits(rng.standard_normal((K, r)).astype(np.float32) * np.float32(2.0 ** -72))
    B = syn.to_bf16_bits(rng.standard_normal((r, N)).astype(np.float32) * np.float32(2.0 ** -72))
    one = lambda v: syn.to_bf16_bits(np.array([v], np.float32))[0]
    A[0, :2] = one(2.0 ** -75)
    A[0, 2:] = 0
    B[:2, 0] = [one(2.0 ** -74), one(2.0 ** -75)]
    B[2:, 0] = 0
    Wb = np.zeros((N, K), np.uint16)
    if base == "nf4":
        w = quantize_gpu(dev_bf16(Wb))
        codes, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16")
        merged = q.qlora_merge_lora(dev_bf16(A), dev_bf16(B), float(r), w=w)
        ref = oracle.merge_lora(A, B, r, float(r), nf4=(codes, q8, s2, N, K))
    else:
        merged = q.qlora_merge_lora(dev_bf16(A), dev_bf16(B), float(r), W=dev_bf16(Wb))
        ref = oracle.merge_lora(A, B, r, float(r), W=Wb)
    torch.cuda.synchronize()
    got = host(merged)
    assert ref[0, 0] == np.float32(2.0 ** -149)
    assert np.count_nonzero(ref) > N * K // 2  # the sums are mostly nonzero subnormals
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "merged weight bits"


def test_merge_zero_adapter_gives_the_dequantized_base():
    N, K, r = 320, 512, 16
    Wb = syn.normal_bf16((N, K), 0.02, 70)
    w = quantize_gpu(dev_bf16(Wb))
    A = dev_bf16(syn.normal_bf16((K, r), 0.1, 71))
    merged = q.qlora_merge_lora(A, torch.zeros((r, N), dtype=torch.bfloat16, device=DEV), 32.0, w=w)
    deq = q.qlora_dequant_bf16(w)
    torch.cuda.synchronize()
    assert torch.equal(merged, deq.float())



# ------------------------------------------------------------------- AdamW
_ADAM = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)


def _adam_gpu_steps(p, m, v, grads, gbf16, want_copy, pinned=False, t0=1):
    """Runs the steps through the C ABI; state on the device, or in pinned
    host memory when `pinned` (the paged optimizer state)."""
    def put(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return t.pin_memory() if pinned else t.to(DEV)
    P, Mm, V = put(p), put(m), put(v)
    pb = torch.empty(p.size, dtype=torch.bfloat16, device=DEV) if want_copy else None
    for i, g in enumerate(grads):
        G = dev_bf16(syn.to_bf16_bits(g)) if gbf16 else torch.from_numpy(g).to(DEV)
        q.qlora_adamw_step(P, G, Mm, V, step=t0 + i, lr=_ADAM["lr"], beta1=_ADAM["beta1"],
                           beta2=_ADAM["beta2"], eps=_ADAM["eps"], weight_decay=_ADAM["wd"],
                           param_bf16=pb)
    torch.cuda.synchronize()
    out = [host(P), host(Mm), host(V)]
    out.append(syn.torch_bf16_to_bits(pb) if want_copy else None)
    return out


def _adam_oracle_steps(p, m, v, grads, gbf16, t0=1):
    pb = None
    for i, g in enumerate(grads):
        gi = syn.to_bf16_bits(g) if gbf16 else g
        p, m, v, pb = oracle.adamw_step(p, gi, m, v, _ADAM["lr"], _ADAM["beta1"], _ADAM["beta2"],
                                        _ADAM["eps"], _ADAM["wd"], t0 + i)
    return p, m, v, pb


def _assert_bits(got, ref, name):
    g = np.ascontiguousarray(got).view(np.uint32 if got.dtype == np.float32 else np.uint16)
    r = np.ascontiguousarray(ref).view(np.uint32 if ref.dtype == np.float32 else np.uint16)
    if not np.array_equal(g, r):
        i = int(np.argmax(g != r))
        raise AssertionError(f"{name}: first difference at {i}: {got[i]!r} vs {ref[i]!r}")


@pytest.mark.parametrize("n,gbf16,copy,steps,t0", [(8, True, True, 1, 1), (1003, True, True, 3, 1),
                                                   (4096 + 5, False, True, 2, 7),
                                                   (777777, True, False, 2, 100),
                                                   (1, False, True, 1, 1)])
def test_adamw_bit_exact(n, gbf16, copy, steps, t0):
    """p, m, v and the bf16 copy bit for bit against the oracle over several
    steps; ragged n (the tail thread's scalar path), both gradient types."""
    say("adamw", n, gbf16, copy, steps, t0)
    p, m, v = syn.adam_state(n, 70 + n % 97)
    grads = [syn.adapter_grad_f32(n, 80 + i) for i in range(steps)]
    got = _adam_gpu_steps(p, m, v, grads, gbf16, copy, t0=t0)
    ref = _adam_oracle_steps(p, m, v, grads, gbf16, t0=t0)
    for k, (a, b) in enumerate(zip(got[:3], ref[:3])):
        _assert_bits(a, b, "pmv"[k])
    if copy:
        _assert_bits(got[3], ref[3], "bf16 copy")


def test_adamw_full_adapter_arena_bit_exact():
    """Every adapter of a Llama-7B decoder at rank 16 (39,976,960 parameters
    in one arena), one step with bf16 gradients, against the oracle."""
    n = syn.adapter_arena_params()
    say("adamw arena", n)
    p, m, v = syn.adam_state(n, 71)
    grads = [syn.adapter_grad_f32(n, 81)]
    got = _adam_gpu_steps(p, m, v, grads, True, True, t0=5)
    ref = _adam_oracle_steps(p, m, v, grads, True, t0=5)
    for k, (a, b) in enumerate(zip(got, ref)):
        _assert_bits(a, b, "pmvb"[k])


def test_adamw_paged_state_in_host_memory():
    """The paged state: master values and moments in pinned host memory,
    stepped by the GPU kernel across the host link, give the same bits."""
    n = 100003
    say("adamw paged", n)
    p, m, v = syn.adam_state(n, 72)
    grads = [syn.adapter_grad_f32(n, 90 + i) for i in range(2)]
    got = _adam_gpu_steps(p, m, v, grads, True, True, pinned=True)
    ref = _adam_oracle_steps(p, m, v, grads, True)
    for k, (a, b) in enumerate(zip(got, ref)):
        _assert_bits(a, b, "pmvb"[k])


def test_adamw_rejects_pageable_host_memory():
    """Memory the device cannot reach is refused before any launch."""
    n = 64
    P = torch.zeros(n, dtype=torch.float32)  # plain pageable host tensor
    G = torch.zeros(n, dtype=torch.float32, device=DEV)
    Mm = torch.zeros(n, dtype=torch.float32, device=DEV)
    V = torch.zeros(n, dtype=torch.float32, device=DEV)
    with pytest.raises(RuntimeError):
        q.qlora_adamw_step(P, G, Mm, V, step=1, lr=1e-3)
    torch.cuda.synchronize()
    assert not P.any()


# ------------------------------------------------ second-level format variants
FMTS = [q.DQ_UINT8, q.DQ_E4M3]


def _check_fmt_roundtrip(Wb, fmt, name):
    w = quantize_gpu(dev_bf16(Wb), fmt)
    codes, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16", fmt)
    assert_nf4_equal(w, codes, q8, s2, name)
    deq = syn.torch_bf16_to_bits(q.qlora_dequant_bf16(w)).ravel()
    assert np.array_equal(deq, oracle.dequant_dq(codes, q8, s2, fmt)[1]), f"{name}: dequant"
    return w


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(1, 64), (3, 192), (257, 640)])
def test_formats_quantize_dequant_bit_exact(fmt, shape):
    say("format quantize", fmt, shape)
    _check_fmt_roundtrip(syn.normal_bf16(shape, 0.02, 300 + shape[0]), fmt, f"fmt {fmt} {shape}")


@pytest.mark.parametrize("fmt", FMTS)
def test_formats_edge_values_and_heavy_tails(fmt):
    """The corner values, and Student-t weights with outliers (blocks whose
    constants sit far below their group's maximum: E4M3 subnormals and small
    integer codes)."""
    say("format edges", fmt)
    _check_fmt_roundtrip(_edge_weights(), fmt, f"fmt {fmt} edges")
    heavy = syn.torch_student_t_outliers_bf16((512, 4096), 301, DEV)
    bits = syn.torch_bf16_to_bits(heavy)
    _check_fmt_roundtrip(bits, fmt, f"fmt {fmt} heavy tails")
    tiny = (syn.normal_f32((64, 1024), 1.0, 302) * np.logspace(-30, 0, 64)[:, None]).astype(np.float32)
    _check_fmt_roundtrip(syn.to_bf16_bits(tiny), fmt, f"fmt {fmt} 30 decades")


@pytest.mark.parametrize("fmt", FMTS)
def test_formats_llama7b_up_bit_exact(fmt):
    N, K = syn.LLAMA7B_TRAIN["weights"]["up"]
    say("format up weight", fmt)
    _check_fmt_roundtrip(syn.normal_bf16((N, K), 0.02, 303), fmt, f"fmt {fmt} up")


@pytest.mark.parametrize("fmt", FMTS)
def test_formats_one_hot_fwd_and_bwd_exact(fmt):
    """One-hot rows through both GEMVs (M = 2 and 4: x slices for two and for
    four tokens; M = 16), the tile kernels (M = 64, 40) and the large-M path
    (M = 600) return the format's dequantized weight
    columns and rows bit for bit: every in-kernel decoding of the absmax
    byte follows the format."""
    N, K, r = 640, 1024, 16
    P = Problem(N, K, r, 32.0, seed=304, fmt=fmt)
    P.Bt = torch.zeros_like(P.Bt)
    Wf = oracle.bf16_to_f32(P.What)
    for M, lean in ((2, False), (4, False), (16, False), (64, False), (600, False), (600, True)):
        ks = np.random.default_rng(M).choice(K, M, replace=False)
        x = np.zeros((M, K), np.uint16)
        x[np.arange(M), ks] = 0x3F80
        assert np.array_equal(host(run_fwd(P, x, lean=lean)), Wf[:, ks].T + 0.0), \
            f"fwd one-hot M={M} lean={lean}"
    for M in (40, 600):
        ns = np.random.default_rng(M + 1).choice(N, M, replace=False)
        dY = np.zeros((M, N), np.uint16)
        dY[np.arange(M), ns] = 0x3F80
        dX, _, _ = run_bwd(P, None, dY, want_grads=False)
        assert np.array_equal(host(dX), Wf[ns] + 0.0), f"bwd one-hot M={M}"


@pytest.mark.parametrize("fmt", FMTS)
def test_formats_layer_within_tolerance(fmt):
    N, K, r = 384, 640, 32
    P = Problem(N, K, r, 16.0, seed=305, fmt=fmt)
    for M in (4, 300):
        x = syn.normal_bf16((M, K), 1.0, 306 + M)
        dY = syn.normal_bf16((M, N), 1.0, 307 + M)
        y = host(run_fwd(P, x))
        yo, _ = oracle.linear_fwd(x, P.What, P.A, P.B, r, 16.0)
        tol_check(y, yo, f"fmt {fmt} y M={M}")
        dX, dA, dB = run_bwd(P, x, dY)
        g = oracle.linear_bwd(x, dY, P.What, P.A, P.B, r, 16.0)
        tol_check(host(dX), g["dX"], f"fmt {fmt} dX M={M}")
        tol_check(host(dA), g["dA"], f"fmt {fmt} dA M={M}")
        tol_check(host(dB), g["dB"], f"fmt {fmt} dB M={M}")


@pytest.mark.parametrize("fmt", FMTS)
def test_formats_merge_and_requantize_bit_exact(fmt):
    N, K, r = 257, 640, 16
    Wb = syn.normal_bf16((N, K), 0.02, 308)
    A = syn.normal_bf16((K, r), 1.0 / np.sqrt(K), 309)
    B = syn.normal_bf16((r, N), 0.01, 310)
    w = quantize_gpu(dev_bf16(Wb), fmt)
    codes, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16", fmt)
    merged = q.qlora_merge_lora(dev_bf16(A), dev_bf16(B), 32.0, w=w)
    ref = oracle.merge_lora(A, B, r, 32.0, nf4=(codes, q8, s2, N, K, fmt))
    torch.cuda.synchronize()
    assert np.array_equal(host(merged).view(np.uint32), ref.view(np.uint32)), "merged bits"
    wq = q.qlora_quantize_nf4_dq(merged, dq_format=fmt)
    assert_nf4_equal(wq, *oracle.quantize_nf4_dq(ref, "f32", fmt), f"fmt {fmt} requantized")
