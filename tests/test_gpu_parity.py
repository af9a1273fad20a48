"""GPU parity: the HIP path through the C ABI against the oracle, element by
element, on seeded inputs.  Integer/byte outputs are bit-exact; floating-point
outputs are within the stated bar (TOL, normwise max relative error)."""

import numpy as np
import pytest

import workloads
from gpu_helpers import (TOL, assert_quant_bit_exact, gpu_layer, normwise_err, oracle_layer, say,
                         dev_bf16, dev_f32, host_bf16_to_f64, oracle_magnitudes, oracle_sampled,
                         rounding_bound_ratio, sweep_blocks)
from oracle import nf4 as onf4
from oracle.bf16 import bits_to_float, float_to_bits

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------
# Quantization: bit-exact indices, packed bytes, scale codes, constants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d_out,d_in", [(256, 256), (64, 320), (128, 192), (4096, 4096)])
def test_quantize_bit_exact(d_out, d_in):
    import nf4_bit_quantized_amd as q
    import torch
    say(f"quantize {d_out}x{d_in}")
    inp = workloads.layer_inputs(d_out, d_in, 1, 1, seed=0, with_dy=False)
    Q = onf4.quantize(inp["W"])
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    torch.cuda.synchronize()
    assert_quant_bit_exact({"packed_h": packed.cpu().numpy(), "codes_h": codes.cpu().numpy(),
                            "consts_h": consts.cpu().numpy()}, Q)


def test_quantize_threshold_sweep_bit_exact():
    """Every NF4 decision threshold and its 40 float32 neighbours on each side,
    in blocks holding a +-1 so that the block scale is 1 and x = w exactly;
    plus all-zero blocks and a ragged last group."""
    import nf4_bit_quantized_amd as q
    import torch
    _, thr = q.qlora_nf4_levels()
    vals = []
    for k in range(15):
        c = np.float32(thr[k])
        vals.append(c)
        for d in (np.float32(np.inf), np.float32(-np.inf)):
            v = c
            for _ in range(40):
                v = np.nextafter(v, d, dtype=np.float32)
                vals.append(v)
    vals += list(onf4.nf4_levels())
    vals = np.array(vals, np.float32)
    per = 63
    nblk = -(-vals.size // per)
    W = np.zeros((nblk, 64), np.float32)
    for b in range(nblk):
        chunk = vals[b * per:(b + 1) * per]
        W[b, 0] = 1.0 if b % 2 == 0 else -1.0
        W[b, 1:1 + chunk.size] = chunk
    W = np.concatenate([W.reshape(-1), np.zeros(64 * 5, np.float32)])     # zero blocks at the end
    pad = (-W.size) % (64 * 64)
    W = np.concatenate([W, np.full(pad, 0.01, np.float32)]).reshape(64, -1)
    say(f"threshold sweep W {W.shape}")
    Q = onf4.quantize(W)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(W))
    torch.cuda.synchronize()
    assert_quant_bit_exact({"packed_h": packed.cpu().numpy(), "codes_h": codes.cpu().numpy(),
                            "consts_h": consts.cpu().numpy()}, Q)


@pytest.mark.parametrize("scales", [
    (0.0123, 0.3, 7.25, 1.0e-3, 2.0 ** -20),
    (1.0e-20, 3.0e-30, 1.0e-38, 1.0e-39, 5.0e-42),     # tiny, down to subnormal block scales
    (1.0e20, 3.0e30, 1.0e38, 3.3e38),                   # huge block scales
])
def test_quantize_threshold_sweep_scaled_bit_exact(scales):
    """The threshold sweep at block scales other than 1, across the float32
    range (subnormal to near the largest finite), with random mantissas."""
    import nf4_bit_quantized_amd as q
    import torch
    _, thr = q.qlora_nf4_levels()
    parts = [sweep_blocks(sc, thr) for sc in scales]
    W = np.concatenate(parts)
    pad = (-W.size) % (64 * 64)
    W = np.concatenate([W, np.zeros(pad, np.float32)]).reshape(64, -1)
    say(f"scaled threshold sweep {scales} W {W.shape}")
    Q = onf4.quantize(W)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(W))
    torch.cuda.synchronize()
    assert_quant_bit_exact({"packed_h": packed.cpu().numpy(), "codes_h": codes.cpu().numpy(),
                            "consts_h": consts.cpu().numpy()}, Q)


def test_quantize_random_magnitudes_bit_exact():
    """Normal weights with each block scaled by 10^u, u uniform in [-44, 38]:
    block scales from subnormal to near the largest float32, mixed in groups."""
    import nf4_bit_quantized_amd as q
    import torch
    rng = np.random.default_rng(11)
    nblk = 64 * 64 * 4
    W = rng.standard_normal((nblk, 64)).astype(np.float32)
    mag = np.power(10.0, rng.uniform(-44.0, 38.0, size=(nblk, 1)))
    W = (W.astype(np.float64) * mag / 4.0).astype(np.float32)
    W = W.reshape(256, -1)
    assert np.all(np.isfinite(W))
    say(f"random magnitudes W {W.shape}")
    Q = onf4.quantize(W)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(W))
    torch.cuda.synchronize()
    assert_quant_bit_exact({"packed_h": packed.cpu().numpy(), "codes_h": codes.cpu().numpy(),
                            "consts_h": consts.cpu().numpy()}, Q)


def test_quantize_deterministic():
    import nf4_bit_quantized_amd as q
    import torch
    inp = workloads.layer_inputs(512, 1024, 1, 1, seed=3, with_dy=False)
    W = dev_f32(inp["W"])
    a = [t.clone() for t in q.qlora_quantize_nf4(W)]
    b = q.qlora_quantize_nf4(W)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# --------------------------------------------------------------------------
# Forward / backward parity
# --------------------------------------------------------------------------

CASES = [
    # (d_out, d_in, T, r, alpha, seed)
    (256, 256, 16, 8, 16.0, 0),       # parity workload: W 256x256, 16 tokens, r=8, alpha=16, seed 0
    (256, 256, 1, 8, 16.0, 1),
    (192, 320, 4, 3, 5.0, 2),         # ragged everything, odd rank
    (128, 256, 17, 16, 32.0, 3),      # first tiled-GEMM size
    (320, 192, 100, 1, 2.0, 4),
    (256, 384, 150, 64, 16.0, 5),
    (448, 256, 64, 128, 64.0, 6),
    (256, 256, 40, 0, 0.0, 7),        # base branch only
    (256, 512, 7, 16, 32.0, 8),       # few-token path, 5..8 tokens
    (128, 448, 12, 8, 16.0, 9),       # few-token path, code runs not 4-byte aligned (K/64 = 7)
    (192, 1024, 16, 64, 16.0, 10),    # few-token path, two stages per contraction slice
    # few-token U split over token groups: four tokens per workgroup with the last
    # group holding one (T = 13, r = 64), two per workgroup with the last holding one
    (256, 512, 13, 64, 16.0, 28),
    (192, 1024, 7, 64, 16.0, 29),
    # few-token kernel with the contraction split over two workgroups (more than
    # four tokens, at most two tiles per workgroup, at least 64 chunks of 128):
    # one tile per run, 65 chunks (ranges of 33 and 32), three tiles per run
    # with the last run two and an odd rank, no rank-r term
    (256, 8192, 16, 64, 16.0, 30),
    (384, 8320, 13, 24, 8.0, 31),
    (4160, 8192, 7, 12, 16.0, 32),
    (512, 8192, 16, 0, 0.0, 33),
    # streaming adapter products (many tokens): ragged token counts, contractions
    # ending in half a 128-chunk, ranks 8 / 24 / 64
    (192, 320, 523, 8, 16.0, 11),
    (256, 192, 600, 24, 8.0, 12),
    (320, 448, 1031, 64, 16.0, 13),
    # U and G over contraction ranges (partials added by a second launch): ranges
    # of unequal length, a short last row tile, ranks 24 and 64
    (4096, 4160, 1000, 24, 8.0, 26),
    (1024, 8192, 1100, 64, 16.0, 27),
    # many tokens with a rank the streaming kernels do not take: split-contraction adapter products
    (192, 384, 1000, 12, 16.0, 24),
    (320, 384, 1000, 12, 16.0, 25),
    # few-token path with several 16-row tiles per workgroup (N/16 above 256)
    (4160, 256, 2, 16, 16.0, 14),     # 2 tiles per workgroup
    (8320, 192, 9, 24, 8.0, 15),      # 3 tiles, the last workgroup 1; K/64 odd
    (16448, 256, 3, 8, 16.0, 16),     # 5 tiles, the last workgroup 3
    (20608, 256, 6, 16, 16.0, 18),    # 6 tiles, the last workgroup 4
    (28736, 128, 16, 64, 16.0, 17),   # 8 tiles, the last workgroup 4
    # one token, more shapes
    (192, 320, 1, 3, 5.0, 20),        # K/64 odd, odd rank
    (320, 4160, 1, 128, 16.0, 21),    # long contraction, largest rank
    (256, 256, 1, 0, 0.0, 22),        # base branch only
    (70016, 512, 1, 16, 16.0, 23),    # 4376 row tiles: eight per workgroup, the last one short
]


@pytest.mark.parametrize("d_out,d_in,T,r,alpha,seed", CASES)
def test_fwd_bwd_parity(d_out, d_in, T, r, alpha, seed):
    """Normwise against the oracle (the bar, 2e-2), and per element within the
    rounding bound of the path (rounding_bound_ratio): c = 2^-10 where the
    restored weight is exact (the tiled products, the adapter products), 2^-7
    for the few-token forward, which scales each block's products by s' in
    fp32 rather than rounding T[q] s' to bf16 per weight."""
    say(f"fwd/bwd d_out={d_out} d_in={d_in} T={T} r={r} alpha={alpha} seed={seed}")
    inp = workloads.layer_inputs(d_out, d_in, T, r, seed)
    o = oracle_layer(inp, r, alpha)
    mag = oracle_magnitudes(inp, r, alpha, Q=o["Q"])
    g = gpu_layer(inp, r, alpha)
    assert_quant_bit_exact(g, o["Q"])
    keys = ["Y", "dX"] + (["U", "dA", "dB"] if r > 0 else [])
    errs = {k: normwise_err(g[k], o[k]) for k in keys}
    bounds = {k: rounding_bound_ratio(g[k], o[k], mag[k], 2.0 ** -7 if (k == "Y" and T <= 16) else 2.0 ** -10)
              for k in keys}
    say("  errors", {k: f"{v:.2e}" for k, v in errs.items()}, "bound ratios", {k: f"{v:.3f}" for k, v in bounds.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    for k, v in bounds.items():
        assert v <= 1.0, (k, v)


@pytest.mark.parametrize("T", [33, 700])
def test_bwd_recomputes_u_when_not_saved(T):
    # 33 tokens: split-contraction adapter kernels; 700: streaming ones
    inp = workloads.layer_inputs(256, 320, T, 8, seed=8)
    a = gpu_layer(inp, 8, 16.0, pass_u=True)
    b = gpu_layer(inp, 8, 16.0, pass_u=False)
    for k in ("dX", "dA", "dB"):
        np.testing.assert_array_equal(a[k], b[k])


def test_attention_shaped_layer_full_size():
    """W 4096x4096, 2048 tokens, r=16, alpha=32: every output against the oracle."""
    (lin,) = workloads.attn_4096()
    say(f"full-size {lin}")
    inp = workloads.layer_inputs(lin.d_out, lin.d_in, lin.T, lin.r, lin.seed)
    o = oracle_layer(inp, lin.r, lin.alpha)
    g = gpu_layer(inp, lin.r, lin.alpha)
    assert_quant_bit_exact(g, o["Q"])
    for k in ("Y", "U", "dX", "dA", "dB"):
        e = normwise_err(g[k], o[k])
        say(f"  {k} err {e:.2e}")
        assert e <= TOL, (k, e)


# --------------------------------------------------------------------------
# Special cases the pages fix
# --------------------------------------------------------------------------

def test_b_zero_equals_base_path_bit_identical():
    """B = 0: the adapter adds nothing -- Y equals the r = 0 result exactly,
    dA = 0 exactly, dB != 0 (A != 0, so B receives a gradient)."""
    import nf4_bit_quantized_amd as q
    import torch
    for T in (8, 64):
        inp = workloads.layer_inputs(256, 192, T, 8, seed=9)
        W = dev_f32(inp["W"])
        packed, codes, consts = q.qlora_quantize_nf4(W)
        X, A, dY = dev_bf16(inp["X"]), dev_bf16(inp["A"]), dev_bf16(inp["dY"])
        B0 = torch.zeros((256, 8), dtype=torch.bfloat16, device="cuda")
        Y, U = q.qlora_linear_fwd(packed, codes, consts, X, A, B0, 16.0)
        Yb, _ = q.qlora_linear_fwd(packed, codes, consts, X, None, None, 0.0)
        dX, dA, dB = q.qlora_linear_bwd(packed, codes, consts, X, A, B0, 16.0, dY, U_in=U)
        dXb, _, _ = q.qlora_linear_bwd(packed, codes, consts, X, None, None, 0.0, dY)
        torch.cuda.synchronize()
        assert torch.equal(Y.float(), Yb.float()), T
        assert torch.all(dA == 0)
        assert dB.abs().max().item() > 0
        assert torch.equal(dX.float(), dXb.float())


def test_sales_tables_bit_exact():
    """The rank-1 and rank-2 sales tables through the layer: W = 0, alpha = r,
    X = identity, so Y = (B A)^T exactly (small integers are exact in bf16)."""
    import nf4_bit_quantized_amd as q
    import torch
    tables = {
        1: ([[10, 20, 30]], [[1, 2, 2, 1]], [[10, 20, 20, 10], [20, 40, 40, 20], [30, 60, 60, 30]]),
        2: ([[10, 20, 30], [1, 0, 2]], [[1, 2, 2, 1], [0, 0, 5, 5]],
            [[10, 20, 25, 15], [20, 40, 40, 20], [30, 60, 70, 40]]),
    }
    for T in (16, 64):                        # few-token path and tiled path
        for r, (cols, rows, want) in tables.items():
            W = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
            packed, codes, consts = q.qlora_quantize_nf4(W)
            B = torch.zeros((64, r), dtype=torch.float32)
            A = torch.zeros((r, 64), dtype=torch.float32)
            for i in range(r):
                B[:3, i] = torch.tensor(cols[i], dtype=torch.float32)
                A[i, :4] = torch.tensor(rows[i], dtype=torch.float32)
            X = torch.zeros((T, 64), dtype=torch.float32)
            X[:min(T, 64), :min(T, 64)] = torch.eye(min(T, 64))
            Y, _ = q.qlora_linear_fwd(packed, codes, consts, X.bfloat16().cuda(), A.bfloat16().cuda(),
                                      B.bfloat16().cuda(), float(r))
            torch.cuda.synchronize()
            got = Y.float().cpu().numpy().T[:3, :4]
            np.testing.assert_array_equal(got, np.array(want, np.float32))
            assert np.linalg.matrix_rank(got) == r


def test_merge_matches_two_branch_result():
    """Y from the layer equals X (W_hat + s B A)^T computed by the oracle."""
    from oracle import lora as olora
    from oracle.bf16 import bits_to_float
    inp = workloads.layer_inputs(256, 256, 48, 16, seed=10)
    g = gpu_layer(inp, 16, 32.0, do_bwd=False)
    W_hat = onf4.dequantize(onf4.quantize(inp["W"]))
    Wm = olora.merged_weight(W_hat, bits_to_float(inp["A"]), bits_to_float(inp["B"]), 32.0, 16)
    want = bits_to_float(inp["X"]) @ Wm.T
    assert normwise_err(g["Y"], want) <= TOL


@pytest.mark.parametrize("d_out,d_in", [(64, 64), (192, 320), (256, 4160), (1024, 1024)])
def test_dequantize_export_bit_exact(d_out, d_in):
    """The exported restored weight equals the oracle's bf16(T[q] s') bit for
    bit ([入门到精通] §3(2)); shapes include a last column tile of 64."""
    import nf4_bit_quantized_amd as q
    import torch
    say(f"dequantize export {d_out}x{d_in}")
    inp = workloads.layer_inputs(d_out, d_in, 1, 1, seed=30)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    W_hat = q.qlora_dequantize_nf4(packed, codes, consts)
    torch.cuda.synchronize()
    got = W_hat.view(torch.int16).cpu().numpy().view(np.uint16)
    want = float_to_bits(onf4.dequantize(onf4.quantize(inp["W"])))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("d_out,d_in,r,alpha", [(128, 128, 8, 16.0), (192, 320, 3, 5.0), (256, 4160, 64, 16.0),
                                                (512, 256, 128, 32.0),
                                                # 512 column blocks: each workgroup walks 4 row tiles
                                                # (next tile's loads in flight), the last block 64 wide
                                                (256, 65472, 24, 8.0)])
def test_merge_export_matches_oracle(d_out, d_in, r, alpha):
    """bf16(W_hat + s B A) ([工程] §3; [X长文] QLoRA section: merged into the
    restored 16-bit weight): every element within one bf16 step of the
    oracle's float64 value rounded to bf16; r = 0 and B = 0 give W_hat exactly."""
    import nf4_bit_quantized_amd as q
    import torch
    from oracle import lora as olora
    say(f"merge export {d_out}x{d_in} r={r}")
    inp = workloads.layer_inputs(d_out, d_in, 1, r, seed=31)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    A, B = dev_bf16(inp["A"]), dev_bf16(inp["B"])
    Wm = q.qlora_merge_lora(packed, codes, consts, A, B, alpha)
    Wh = q.qlora_dequantize_nf4(packed, codes, consts)
    W0 = q.qlora_merge_lora(packed, codes, consts, A, torch.zeros_like(B), alpha)
    torch.cuda.synchronize()
    assert torch.equal(W0.view(torch.int16), Wh.view(torch.int16))
    W_hat = onf4.dequantize(onf4.quantize(inp["W"]))
    want = olora.merged_weight(W_hat, bits_to_float(inp["A"]), bits_to_float(inp["B"]), alpha, r)
    got = host_bf16_to_f64(Wm)
    # one bf16 step at the value's magnitude (8 significant bits), plus the
    # fp32 rounding of the two terms (which matters only where they cancel)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
    tol = step + 2.0 ** -20 * (np.abs(W_hat) + np.abs(want - W_hat))
    worst = float(np.max(np.abs(got - want) / tol))
    say(f"  worst error {worst:.3f} of the bound")
    assert worst <= 1.0
    assert not torch.equal(Wm.view(torch.int16), Wh.view(torch.int16))


def test_deterministic_fwd_bwd():
    inp = workloads.layer_inputs(256, 512, 80, 16, seed=11)
    a = gpu_layer(inp, 16, 32.0)
    b = gpu_layer(inp, 16, 32.0)
    for k in ("Y", "U", "dX", "dA", "dB"):
        np.testing.assert_array_equal(a[k], b[k])
    a = gpu_layer(workloads.layer_inputs(256, 512, 8, 16, seed=11), 16, 32.0)
    b = gpu_layer(workloads.layer_inputs(256, 512, 8, 16, seed=11), 16, 32.0)
    for k in ("Y", "U", "dX", "dA", "dB"):
        np.testing.assert_array_equal(a[k], b[k])


def test_workspace_reuse_across_calls():
    """One workspace shared by forward and backward calls of several sizes
    (its contents left over from the previous call) gives the same outputs as
    a fresh workspace, bit for bit."""
    import nf4_bit_quantized_amd as q
    import torch
    shapes = [(256, 384, 150, 64), (448, 256, 64, 16), (4096, 1024, 600, 16), (256, 256, 16, 8)]
    size = max(max(q.qlora_fwd_workspace_bytes(n, k, t, r), q.qlora_bwd_workspace_bytes(n, k, t, r))
               for (n, k, t, r) in shapes)
    ws = torch.full((size,), 0x5A, dtype=torch.uint8, device="cuda")   # stale contents
    for rep in range(2):
        for (n, k, t, r) in shapes:
            say(f"workspace reuse {n}x{k} T={t} r={r} pass {rep}")
            inp = workloads.layer_inputs(n, k, t, r, seed=21)
            packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
            X, A, B, dY = (dev_bf16(inp[key]) for key in ("X", "A", "B", "dY"))
            Y1, U1 = q.qlora_linear_fwd(packed, codes, consts, X, A, B, 16.0, workspace=ws)
            g1 = q.qlora_linear_bwd(packed, codes, consts, X, A, B, 16.0, dY, U_in=U1, workspace=ws)
            Y2, U2 = q.qlora_linear_fwd(packed, codes, consts, X, A, B, 16.0)
            g2 = q.qlora_linear_bwd(packed, codes, consts, X, A, B, 16.0, dY, U_in=U2)
            torch.cuda.synchronize()
            assert torch.equal(Y1, Y2) and torch.equal(U1, U2)
            for a, b in zip(g1, g2):
                assert torch.equal(a, b)


def test_few_tokens_with_unaligned_codes():
    """Codes off a 16-byte boundary: the few-token forward runs the tiled kernel
    instead of the weight-streaming one; both results match the oracle."""
    import nf4_bit_quantized_amd as q
    import torch
    for T in (1, 4):
        inp = workloads.layer_inputs(256, 320, T, 8, seed=21)
        o = oracle_layer(inp, 8, 16.0, do_bwd=False)
        packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
        buf = torch.zeros(codes.numel() + 16, dtype=torch.uint8, device="cuda")
        shifted = buf[1:1 + codes.numel()]
        shifted.copy_(codes)
        X, A, B = dev_bf16(inp["X"]), dev_bf16(inp["A"]), dev_bf16(inp["B"])
        for c in (codes, shifted):
            Y, _ = q.qlora_linear_fwd(packed, c, consts, X, A, B, 16.0)
            torch.cuda.synchronize()
            e = normwise_err(host_bf16_to_f64(Y), o["Y"])
            say(f"  T={T} codes offset {c.data_ptr() % 16}: Y err {e:.2e}")
            assert e <= TOL, (T, e)


@pytest.mark.parametrize("d_out,d_in,T,split", [
    (256, 8192, 16, True),     # one tile per workgroup, 64 chunks
    (384, 8320, 13, True),     # 65 chunks
    (8192, 8192, 5, True),     # two tiles per workgroup unsplit
    (256, 8192, 4, False),     # four tokens or fewer: one launch
    (256, 4096, 16, False),    # fewer than 64 chunks
    (8320, 8192, 16, False),   # three tiles per workgroup
])
def test_few_token_contraction_split_launches(d_out, d_in, T, split):
    """The few-token forward splits the contraction over two workgroups (and
    adds the ranges in a second launch) exactly for more than four tokens, at
    most two tiles per workgroup and at least 64 chunks of 128 weights; the
    parity cases above check the values of both forms against the oracle."""
    import nf4_bit_quantized_amd as q
    import torch
    say(f"decode split d_out={d_out} d_in={d_in} T={T} expect split={split}")
    g = torch.Generator(device="cuda").manual_seed(5)
    packed, codes, consts = q.qlora_quantize_nf4(torch.randn(d_out, d_in, device="cuda", generator=g) * 0.02)
    X = torch.randn(T, d_in, device="cuda", generator=g).to(torch.bfloat16)
    A = (torch.randn(16, d_in, device="cuda", generator=g) / 16).to(torch.bfloat16)
    B = (torch.randn(d_out, 16, device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    q.qlora_trace_select({"decode", "decode_sum"})
    q.qlora_trace_read(reset=True)
    try:
        q.qlora_linear_fwd(packed, codes, consts, X, A, B, 32.0)
        torch.cuda.synchronize()
        t = q.qlora_trace_read(reset=True)
    finally:
        q.qlora_trace_enable(False)
    assert t.get("decode", (0, 0.0))[0] == 1, t
    assert t.get("decode_sum", (0, 0.0))[0] == (1 if split else 0), t


def test_zero_tokens_is_a_no_op():
    import nf4_bit_quantized_amd as q
    import torch
    inp = workloads.layer_inputs(128, 128, 0, 4, seed=12)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    X = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    A, B = dev_bf16(inp["A"]), dev_bf16(inp["B"])
    Y, U = q.qlora_linear_fwd(packed, codes, consts, X, A, B, 8.0)
    dA = torch.full((4, 128), 7.0, device="cuda")
    dB = torch.full((128, 4), 7.0, device="cuda")
    q.qlora_linear_bwd(packed, codes, consts, X, A, B, 8.0, dY, dA=dA, dB=dB)
    torch.cuda.synchronize()
    assert Y.shape == (0, 128) and torch.all(dA == 0) and torch.all(dB == 0)


def test_restore_is_bit_exact_through_identity():
    """With X = I (forward, r = 0) every output is one restored weight, so Y
    must equal W_hat^T bit for bit; with dY = I the same holds for dX = W_hat.
    Covers the tiled forward and the transposed-restore dX.  The few-token
    path applies the block scale to the product of bf16(T[q]) instead of
    rounding T[q] * s' to bf16 first, so there each restored weight must lie
    within two bf16 rounding steps (relative 2^-7) of W_hat, zeros exact."""
    import nf4_bit_quantized_amd as q
    import torch
    d_out, d_in = 320, 256
    inp = workloads.layer_inputs(d_out, d_in, 1, 1, seed=13, with_dy=False)
    W_hat = onf4.dequantize(onf4.quantize(inp["W"]))            # float32, bf16-valued
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    eye_k = torch.eye(d_in, dtype=torch.bfloat16, device="cuda")
    Y, _ = q.qlora_linear_fwd(packed, codes, consts, eye_k, None, None, 0.0)
    eye_n = torch.eye(d_out, dtype=torch.bfloat16, device="cuda")
    dX, _, _ = q.qlora_linear_bwd(packed, codes, consts, torch.zeros((d_out, d_in), dtype=torch.bfloat16,
                                                                      device="cuda"), None, None, 0.0, eye_n)
    Y16, _ = q.qlora_linear_fwd(packed, codes, consts, eye_k[:16].contiguous(), None, None, 0.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Y.float().cpu().numpy(), W_hat.T)
    np.testing.assert_array_equal(dX.float().cpu().numpy(), W_hat)
    got16, ref16 = Y16.float().cpu().numpy(), W_hat.T[:16]
    assert np.all(np.abs(got16 - ref16) <= np.float32(2.0 ** -7) * np.abs(ref16))


# --------------------------------------------------------------------------
# Full-size decode shapes: 8192 <-> 28672, T in {1, 4, 16}, r = 64, alpha = 16
# --------------------------------------------------------------------------

def _oracle_rows(W, rows, K):
    """Restored rows of W (float64) and their packed bytes, codes and group
    constants, from the oracle quantizing only the 256-block groups that cover
    each row (groups start at multiples of 16384 weights, so they match the
    full-tensor quantization exactly)."""
    out = {}
    flat = W.reshape(-1)
    for n in rows:
        a, b = n * K, (n + 1) * K
        g0, g1 = a // 16384, -(-b // 16384)
        seg = flat[g0 * 16384: min(g1 * 16384, flat.size)]
        Q = onf4.quantize(seg.reshape(1, -1))
        Wh = onf4.dequantize(Q).reshape(-1)
        lo = a - g0 * 16384
        out[n] = {
            "w": Wh[lo: lo + K].astype(np.float64),
            "packed": Q.packed.reshape(-1)[lo // 2: (lo + K) // 2],
            "codes": Q.codes[lo // 64: (lo + K) // 64],
            "consts": (g0, Q.consts),
        }
    return out


@pytest.mark.parametrize("d_out,d_in", [(28672, 8192), (8192, 28672)])
def test_decode_full_size_sampled(d_out, d_in):
    """The few-token forward at the decode shapes, T = 1, 4, 16: sampled output
    columns against the oracle (normwise 2e-2), and the sampled rows' packed
    bytes, codes and group constants bit-exact."""
    import nf4_bit_quantized_amd as q
    import torch
    from oracle.bf16 import bits_to_float
    r, alpha = 64, 16.0
    say(f"decode full size {d_out}x{d_in}: drawing inputs")
    inp = workloads.layer_inputs(d_out, d_in, 16, r, seed=3, with_dy=False)
    rng = np.random.default_rng(7)
    rows = sorted(rng.choice(d_out, size=48, replace=False).tolist())
    ref = _oracle_rows(inp["W"], rows, d_in)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    pk = packed.view(-1)
    cd = codes.view(-1)
    for n in rows:
        assert np.array_equal(pk[n * d_in // 2:(n + 1) * d_in // 2].cpu().numpy(), ref[n]["packed"]), n
        assert np.array_equal(cd[n * d_in // 64:(n + 1) * d_in // 64].cpu().numpy(), ref[n]["codes"]), n
        g0, cs = ref[n]["consts"]
        assert np.array_equal(consts[g0:g0 + cs.size].cpu().numpy().view(np.uint32), cs.view(np.uint32)), n
    X = bits_to_float(inp["X"]).astype(np.float64)
    A = bits_to_float(inp["A"]).astype(np.float64)
    B = bits_to_float(inp["B"]).astype(np.float64)
    s = float(np.float32(alpha / r))
    Wrows = np.stack([ref[n]["w"] for n in rows])                      # [rows][K]
    for T in (1, 4, 16):
        say(f"  T={T}")
        Xg = dev_bf16(inp["X"][:T])
        Y, _ = q.qlora_linear_fwd(packed, codes, consts, Xg, dev_bf16(inp["A"]), dev_bf16(inp["B"]), alpha)
        torch.cuda.synchronize()
        got = Y.float().cpu().numpy()[:, rows].astype(np.float64)
        U = X[:T] @ A.T
        want = X[:T] @ Wrows.T + s * (U @ B[rows].T)
        err = np.max(np.abs(got - want)) / np.max(np.abs(want))
        say(f"    normwise error {err:.2e}")
        assert err <= TOL, (T, err)


# --------------------------------------------------------------------------
# Full-size training shapes: the MLP set (4096 <-> 11008) and the 65B-class
# projections (8192 x 8192, 8192 <-> 22016), 4096 tokens, r = 64, alpha = 16
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d_out,d_in", [(11008, 4096), (4096, 11008), (8192, 8192), (22016, 8192), (8192, 22016)])
def test_training_shapes_full_size_sampled(d_out, d_in):
    """Quantize bit-exact over the whole weight; forward and backward at the
    full size with sampled outputs against the oracle: Y and dB on 32 sampled
    output rows, dX and dA on 32 sampled input columns (normwise 2e-2)."""
    import nf4_bit_quantized_amd as q
    import torch
    from oracle.bf16 import bits_to_float
    T, r, alpha = 4096, 64, 16.0
    say(f"training shape {d_out}x{d_in}, T={T}: drawing inputs")
    inp = workloads.layer_inputs(d_out, d_in, T, r, seed=100 + d_out % 97)
    Q = onf4.quantize(inp["W"])
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    torch.cuda.synchronize()
    assert_quant_bit_exact({"packed_h": packed.cpu().numpy(), "codes_h": codes.cpu().numpy(),
                            "consts_h": consts.cpu().numpy()}, Q)
    say("  quantize bit-exact")
    Xg, Ag, Bg, dYg = (dev_bf16(inp[k]) for k in ("X", "A", "B", "dY"))
    Y, U = q.qlora_linear_fwd(packed, codes, consts, Xg, Ag, Bg, alpha)
    dX, dA, dB = q.qlora_linear_bwd(packed, codes, consts, Xg, Ag, Bg, alpha, dYg, U_in=U)
    torch.cuda.synchronize()

    rng = np.random.default_rng(d_out * 7 + d_in)
    rows = np.sort(rng.choice(d_out, size=32, replace=False))
    cols = np.sort(rng.choice(d_in, size=32, replace=False))
    X, A, B, dY = (bits_to_float(inp[k]) for k in ("X", "A", "B", "dY"))
    want = oracle_sampled(Q, X, A, B, dY, alpha, r, rows, cols)
    ri, ci = torch.as_tensor(rows, device="cuda"), torch.as_tensor(cols, device="cuda")
    got = {
        "Y": Y.index_select(1, ri).float().cpu().numpy().astype(np.float64),
        "dB": dB.index_select(0, ri).cpu().numpy().astype(np.float64),
        "dX": dX.index_select(1, ci).float().cpu().numpy().astype(np.float64),
        "dA": dA.index_select(1, ci).cpu().numpy().astype(np.float64),
    }
    errs = {k: float(np.max(np.abs(got[k] - want[k])) / np.max(np.abs(want[k]))) for k in want}
    say("  errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)
