"""GPU parity of the grouped forward (one quantize kernel + one contraction
kernel over many problems), including the full 70B-shaped decode sweep in the
launch configuration the benchmark times, checked on sampled matrices."""
import os

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_y_close, bl, pack_weights, say, torch_cuda
from ternary_weight_linear_fwd_amd import synthetic as S

pytestmark = pytest.mark.gpu
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.mark.parametrize("M", [1, 3, 8, 16, 40, 64, 96])
def test_grouped_block_matches_oracle(M):
    torch = torch_cuda()
    L = bl()
    specs, refs = [], []
    shared_x = torch.from_numpy(S.c2_x(S.C2_PROJS[0], M)).cuda()     # q, k, v share one input
    shared_xq = torch.empty((M, 3200), dtype=torch.int8, device="cuda")
    shared_eta = torch.empty(M, dtype=torch.float32, device="cuda")
    for p in S.C2_PROJS:
        W = S.c2_weight(p)
        packed, g = pack_weights(W)
        Wt, _ = oracle.quantize_weights(W)
        if p.name in ("q", "k", "v"):
            x_np, x, xq, eta = S.c2_x(S.C2_PROJS[0], M), shared_x, shared_xq, shared_eta
        else:
            x_np = S.c2_x(p, M)
            x = torch.from_numpy(x_np).cuda()
            xq = torch.empty((M, p.K), dtype=torch.int8, device="cuda")
            eta = torch.empty(M, dtype=torch.float32, device="cuda")
        y = torch.empty((M, p.N), dtype=torch.float32, device="cuda")
        y_int = torch.empty((M, p.N), dtype=torch.int32, device="cuda")
        specs.append(dict(x=x, xq=xq, eta=eta, packed=packed, y=y, y_int=y_int, gamma=g, N=p.N, K=p.K))
        refs.append((x_np, Wt, g))
    probs = L.make_problems(specs)
    tb = L.bitlinear_grouped_table_bytes(probs, len(specs), M)
    table = torch.empty(tb, dtype=torch.uint8, device="cuda")
    plan = L.bitlinear_grouped_plan_init(probs, len(specs), M, table, tb)
    assert plan.quant_rows == 5 * M          # q/k/v quantized once
    for rep in range(2):                      # a second run gives the same bits
        L.bitlinear_forward_grouped(plan)
        torch.cuda.synchronize()
        for s, (x_np, Wt, g) in zip(specs, refs):
            y_ref, xq_ref, eta_ref, y_int_ref = oracle.forward(x_np, Wt, g, threads=THREADS)
            assert np.array_equal(s["y_int"].cpu().numpy(), y_int_ref)
            y = s["y"].cpu().numpy()
            assert_y_close(y, y_ref)
            assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))


SAMPLES = [(0, "q"), (17, "k"), (33, "v"), (42, "gate"), (63, "o"), (79, "down")]


@pytest.mark.timeout(900)
def test_c4_sweep_full_size_sampled():
    torch = torch_cuda()
    from ternary_weight_linear_fwd_amd.sweep import DecodeSweep
    sw = DecodeSweep(Ms=(1, 16), keep_int=SAMPLES, progress=say)
    assert sw.weight_bytes() == 17_112_760_320
    for M in (1, 16):
        sw.step(M)
    torch.cuda.synchronize()
    projs = {p.name: p for p in S.C4_PROJS}
    for layer, name in SAMPLES:
        p = projs[name]
        say(f"C4 check layer={layer} {name} ({p.K}->{p.N})")
        W = S.c4_weight_device(layer, p).cpu().numpy()
        Wt, g = oracle.quantize_weights(W)
        del W
        assert np.float32(sw.gamma[(layer, name)]) == g
        for M in (1, 16):
            key = (layer, name, M)
            x = sw.x[key].cpu().numpy()
            y_ref, xq_ref, eta_ref, y_int_ref = oracle.forward(x, Wt, g, threads=THREADS)
            assert np.array_equal(sw.xq[key].cpu().numpy(), xq_ref)
            assert np.array_equal(sw.y_int[key].cpu().numpy(), y_int_ref)
            y = sw.y[key].cpu().numpy()
            assert_y_close(y, y_ref)
            assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))


# Rows of very different lengths in one plan: K past the quantizer's register
# budget (32768 floats: read twice), tiny K, and ordinary K; x̃ and eta from the
# grouped quantizer and the integer sums bit-exact.
@pytest.mark.parametrize("M", [2, 20])
def test_grouped_mixed_row_lengths(M):
    torch = torch_cuda()
    L = bl()
    shapes = [(128, 33792), (200, 64), (70, 16), (96, 4160)]
    specs, refs = [], []
    for i, (N, K) in enumerate(shapes):
        x_np = S.random_x(900 + 10 * M + i, M, K, "t3")
        Wt = S.random_ternary(950 + i, N, K)
        packed = torch.empty(L.bitlinear_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
        L.bitlinear_pack_ternary(torch.from_numpy(Wt).cuda(), N, K, packed)
        xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
        eta = torch.empty(M, dtype=torch.float32, device="cuda")
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        y_int = torch.empty((M, N), dtype=torch.int32, device="cuda")
        specs.append(dict(x=torch.from_numpy(x_np).cuda(), xq=xq, eta=eta, packed=packed, y=y, y_int=y_int,
                          gamma=np.float32(0.03), N=N, K=K))
        refs.append((x_np, Wt))
    probs = L.make_problems(specs)
    tb = L.bitlinear_grouped_table_bytes(probs, len(specs), M)
    table = torch.empty(tb, dtype=torch.uint8, device="cuda")
    plan = L.bitlinear_grouped_plan_init(probs, len(specs), M, table, tb)
    L.bitlinear_forward_grouped(plan)
    torch.cuda.synchronize()
    for s, (x_np, Wt) in zip(specs, refs):
        say(f"mixed rows M={M} N={s['N']} K={s['K']}")
        y_ref, xq_ref, eta_ref, y_int_ref = oracle.forward(x_np, Wt, np.float32(0.03), threads=THREADS)
        assert np.array_equal(s["xq"].cpu().numpy(), xq_ref)
        assert np.array_equal(s["eta"].cpu().numpy().view(np.uint32), eta_ref.view(np.uint32))
        assert np.array_equal(s["y_int"].cpu().numpy(), y_int_ref)
        assert np.array_equal(s["y"].cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


# A small grouped plan (too few row blocks to fill the chip) splits long K
# loops: in the dot4 GEMV up to 4 tokens, the streaming MFMA kernel up to 16,
# 64 x 256 prefill tiles above.  Problems whose K gives one to many slices (a 16-k problem stays
# whole), ragged M, N and K, run twice on the same table.
@pytest.mark.parametrize("M", [2, 4, 12, 24, 64, 65, 128, 200])
def test_grouped_split_k_small_plan(M):
    torch = torch_cuda()
    L = bl()
    shapes = [(300, 4160), (64, 16), (1000, 11008), (257, 2064)]
    specs, refs = [], []
    for i, (N, K) in enumerate(shapes):
        say(f"grouped split plan M={M} problem {i}: N={N} K={K}")
        x_np = S.random_x(900 + 10 * i + M, M, K, "t3")
        Wt = S.random_ternary(901 + 10 * i, N, K)
        g = np.float32(0.0131 + 0.001 * i)
        packed = torch.empty(L.bitlinear_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
        L.bitlinear_pack_ternary(torch.from_numpy(Wt).cuda(), N, K, packed)
        specs.append(dict(x=torch.from_numpy(x_np).cuda(), xq=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                          eta=torch.empty(M, dtype=torch.float32, device="cuda"), packed=packed,
                          y=torch.empty((M, N), dtype=torch.float32, device="cuda"),
                          y_int=torch.empty((M, N), dtype=torch.int32, device="cuda"), gamma=g, N=N, K=K))
        refs.append((x_np, Wt, g))
    probs = L.make_problems(specs)
    tb = L.bitlinear_grouped_table_bytes(probs, len(specs), M)
    table = torch.empty(tb, dtype=torch.uint8, device="cuda")
    plan = L.bitlinear_grouped_plan_init(probs, len(specs), M, table, tb)
    # split: more work units than row blocks (64 rows per unit for the
    # dot4 GEMV, 256 otherwise), and the partials in the table
    width = 64 if M <= 4 else 256
    assert plan.units > sum((N + width - 1) // width for N, _ in shapes)
    assert tb >= plan.units * M * width * 4
    for rep in range(2):
        L.bitlinear_forward_grouped(plan)
        torch.cuda.synchronize()
        for s, (x_np, Wt, g) in zip(specs, refs):
            y_ref, _, _, y_int_ref = oracle.forward(x_np, Wt, g, threads=THREADS)
            assert np.array_equal(s["y_int"].cpu().numpy(), y_int_ref)
            assert np.array_equal(s["y"].cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


# A grouped plan past 64 tokens with enough 256-column blocks to fill the
# chip takes the 128 x 256 prefill tiles; a small one with short K loops the
# 64 x 256 tiles without split: ragged N (whole waves past N), K with tail
# blocks, own row sums per tile.
@pytest.mark.parametrize("M,shapes", [(130, [(33000, 80), (32832, 208), (300, 1040)]),
                                      (200, [(33000, 80), (32832, 208), (300, 1040)]),
                                      (100, [(2000, 80), (1500, 208), (300, 1008)])])
def test_grouped_prefill_tiles(M, shapes):
    torch = torch_cuda()
    L = bl()
    specs, refs = [], []
    for i, (N, K) in enumerate(shapes):
        say(f"grouped prefill M={M} problem {i}: N={N} K={K}")
        x_np = S.random_x(700 + 10 * i + M, M, K, "t3")
        Wt = S.random_ternary(701 + 10 * i, N, K)
        g = np.float32(0.021 + 0.002 * i)
        packed = torch.empty(L.bitlinear_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
        L.bitlinear_pack_ternary(torch.from_numpy(Wt).cuda(), N, K, packed)
        specs.append(dict(x=torch.from_numpy(x_np).cuda(), xq=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                          eta=torch.empty(M, dtype=torch.float32, device="cuda"), packed=packed,
                          y=torch.empty((M, N), dtype=torch.float32, device="cuda"),
                          y_int=torch.empty((M, N), dtype=torch.int32, device="cuda"), gamma=g, N=N, K=K))
        refs.append((x_np, Wt, g))
    probs = L.make_problems(specs)
    tb = L.bitlinear_grouped_table_bytes(probs, len(specs), M)
    table = torch.empty(tb, dtype=torch.uint8, device="cuda")
    plan = L.bitlinear_grouped_plan_init(probs, len(specs), M, table, tb)
    assert plan.units == sum((N + 255) // 256 for N, _ in shapes)   # one unit per 256 columns
    L.bitlinear_forward_grouped(plan)
    torch.cuda.synchronize()
    for s, (x_np, Wt, g) in zip(specs, refs):
        y_ref, _, _, y_int_ref = oracle.forward(x_np, Wt, g, threads=THREADS)
        assert np.array_equal(s["y_int"].cpu().numpy(), y_int_ref)
        assert np.array_equal(s["y"].cpu().numpy().view(np.uint32), y_ref.view(np.uint32))
