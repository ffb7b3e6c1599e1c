"""GPU parity of the grouped forward (one quantize kernel + one contraction
kernel over many problems), including the full 70B-shaped decode sweep in the
launch configuration the benchmark times, checked on sampled matrices."""
import os

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_y_close, bl, near_tie_rows, pack_weights, say, torch_cuda
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
    if M <= 4:   # fused: every workgroup quantizes its own rows, no quantize stage
        assert plan.quant_rows == 0 and plan.units == sum((p.N + 63) // 64 for p in S.C2_PROJS)
    else:
        assert plan.quant_rows == 5 * M      # q/k/v quantized once
    for rep in range(2):                      # a second run gives the same bits
        for s in specs:
            s["xq"].fill_(99)
            s["eta"].fill_(-1.0)
        L.bitlinear_forward_grouped(plan)
        torch.cuda.synchronize()
        for s, (x_np, Wt, g) in zip(specs, refs):
            y_ref, xq_ref, eta_ref, y_int_ref = oracle.forward(x_np, Wt, g, threads=THREADS)
            assert np.array_equal(s["xq"].cpu().numpy(), xq_ref)
            assert np.array_equal(s["eta"].cpu().numpy().view(np.uint32), eta_ref.view(np.uint32))
            assert np.array_equal(s["y_int"].cpu().numpy(), y_int_ref)
            y = s["y"].cpu().numpy()
            assert_y_close(y, y_ref)
            assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))


# One matrix from every band of ten layers, every projection kind at least once.
SAMPLES = [(0, "q"), (17, "k"), (25, "up"), (33, "v"), (42, "gate"), (56, "up"), (63, "o"), (79, "down")]


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


@pytest.mark.timeout(900)
def test_c4_sweep_base3_full_size_sampled():
    # the same 70B-shaped sweep with every matrix in the base-3 layout, at one
    # and eight tokens, as bench.py times it
    torch = torch_cuda()
    from ternary_weight_linear_fwd_amd.sweep import DecodeSweep
    sw = DecodeSweep(Ms=(), formats=("base3",), base3_Ms=(1, 8), keep_int=SAMPLES, progress=say)
    assert sw.weight_bytes("base3") == 13_754_695_680
    for M in (1, 8):
        sw.step(M, fmt="base3")
    torch.cuda.synchronize()
    projs = {p.name: p for p in S.C4_PROJS}
    for layer, name in SAMPLES:
        p = projs[name]
        say(f"C4 base-3 check layer={layer} {name} ({p.K}->{p.N})")
        W = S.c4_weight_device(layer, p).cpu().numpy()
        Wt, g = oracle.quantize_weights(W)
        del W
        assert np.float32(sw.gamma[(layer, name)]) == g
        for M in (1, 8):
            key = (layer, name, M)
            x = sw.x[key].cpu().numpy()
            y_ref, xq_ref, eta_ref, y_int_ref = oracle.forward(x, Wt, g, threads=THREADS)
            assert np.array_equal(sw.xq[key].cpu().numpy(), xq_ref)
            assert np.array_equal(sw.y_int[key].cpu().numpy(), y_int_ref)
            assert np.array_equal(sw.y[key].cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


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
# loops: in the dot4 GEMV up to 4 tokens (where some K is past the fused
# kernel's 16384), the streaming MFMA kernel up to 16, 64 x 256 prefill
# tiles above.  Problems whose K gives one to many slices (a 16-k problem
# stays whole), ragged M, N and K, run twice on the same table.
@pytest.mark.parametrize("M,long_k", [(2, False), (4, False), (3, True), (4, True), (12, False), (24, False),
                                      (64, False), (65, False), (128, False), (200, False)])
def test_grouped_split_k_small_plan(M, long_k):
    torch = torch_cuda()
    L = bl()
    shapes = [(300, 4160), (64, 16), (1000, 11008), (257, 2064)] + ([(200, 20480)] if long_k else [])
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
    # dot4 GEMV, 256 otherwise), and the partials in the table; up to four
    # tokens with every K at most 16384 the fused kernel takes whole K loops
    width = 64 if M <= 4 else 256
    if M <= 4 and not long_k:
        assert plan.units == sum((N + 63) // 64 for N, _ in shapes) and plan.quant_rows == 0
    else:
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


# The fused small-plan decode (M <= 4: quantize, whole-K contraction and
# dequant in one launch): problems fed from float32 rows and from already
# quantized ones in one plan, a shared float32 input, ragged N, K with tail
# blocks, the longest K the fused kernel takes (16384) and the shortest (16),
# all-zero rows, int8 extremes; x~, eta, y_int and y against the oracle, twice.
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_grouped_fused_decode(M):
    torch = torch_cuda()
    L = bl()
    # the longest K the fused kernel takes: 16384, or what its 56 KB of x~ rows allow
    shapes = [(300, 4144), (64, 16), (1000, 16384 if M <= 3 else 14336), (257, 2064), (130, 1040), (65, 1040)]
    xs = {K: S.random_x(400 + K + M, M, K, "t3") for _, K in shapes}
    xs[2064][0] = 0.0                                     # an all-zero row
    xs[16][M - 1] = np.float32(3.0e38) * (np.arange(16) % 2 * 2 - 1)   # |x| at the float32 top
    shared = {K: torch.from_numpy(v).cuda() for K, v in xs.items()}
    xq_shared = torch.empty((M, 1040), dtype=torch.int8, device="cuda")
    eta_shared = torch.empty(M, dtype=torch.float32, device="cuda")
    specs, refs = [], []
    for i, (N, K) in enumerate(shapes):
        say(f"fused decode M={M} problem {i}: N={N} K={K}")
        Wt = S.random_ternary(500 + i, N, K)
        g = np.float32(0.017 + 0.003 * i)
        packed = torch.empty(L.bitlinear_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
        L.bitlinear_pack_ternary(torch.from_numpy(Wt).cuda(), N, K, packed)
        x_np = xs[K]
        xq_ref, eta_ref = oracle.quantize_act(x_np)
        if i == 3:   # already quantized: x = NULL, x~ and eta given
            x, xq, eta = None, torch.from_numpy(xq_ref).cuda(), torch.from_numpy(eta_ref).cuda()
        elif K == 1040:   # two problems share one float32 input and its x~ / eta buffers
            x, xq, eta = shared[K], xq_shared, eta_shared
        else:
            x = shared[K]
            xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
            eta = torch.empty(M, dtype=torch.float32, device="cuda")
        specs.append(dict(x=x, xq=xq, eta=eta, packed=packed,
                          y=torch.empty((M, N), dtype=torch.float32, device="cuda"),
                          y_int=torch.empty((M, N), dtype=torch.int32, device="cuda"), gamma=g, N=N, K=K))
        refs.append((x_np, Wt, g, xq_ref, eta_ref))
    probs = L.make_problems(specs)
    tb = L.bitlinear_grouped_table_bytes(probs, len(specs), M)
    table = torch.empty(tb, dtype=torch.uint8, device="cuda")
    plan = L.bitlinear_grouped_plan_init(probs, len(specs), M, table, tb)
    assert plan.quant_rows == 0 and plan.units == sum((N + 63) // 64 for N, _ in shapes)
    for rep in range(2):
        L.bitlinear_forward_grouped(plan)
        torch.cuda.synchronize()
        for s, (x_np, Wt, g, xq_ref, eta_ref) in zip(specs, refs):
            y_ref, y_int_ref = oracle.forward_q(xq_ref, eta_ref, Wt, g, threads=THREADS)
            assert np.array_equal(s["xq"].cpu().numpy(), xq_ref)
            assert np.array_equal(s["eta"].cpu().numpy().view(np.uint32), eta_ref.view(np.uint32))
            assert np.array_equal(s["y_int"].cpu().numpy(), y_int_ref)
            assert np.array_equal(s["y"].cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


# The planner's unit order (no forward runs): unsplit plans run each XCD's
# run of the grid longest K loop first, stably (a problem's units stay in
# order), plans whose kernel takes units in grid order (the fused decode) are
# one such run, and split plans keep problem, block, slice order.  The table
# is read back and checked against these rules and against the full set of
# (problem, unit) pairs.
def _plan_units(L, torch, shapes, M, fmt):
    dummy = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    base = dummy.data_ptr()
    specs = [dict(x=None, xq=base, eta=base, packed=base, y=base, gamma=1.0, N=N, K=K, format=fmt)
             for N, K in shapes]
    probs = L.make_problems(specs)
    tb = L.bitlinear_grouped_table_bytes(probs, len(specs), M)
    table = torch.empty(tb, dtype=torch.uint8, device="cuda")
    plan = L.bitlinear_grouped_plan_init(probs, len(specs), M, table, tb)
    torch.cuda.synchronize()
    off = -(-len(specs) * 80 // 256) * 256           # units follow the 80-byte problem descriptors
    raw = table.cpu().numpy()[off:off + 8 * plan.units].view(np.int32).reshape(-1, 2)
    return plan, [tuple(int(v) for v in u) for u in raw]


def _xcd_runs(n, per):
    T = -(-n // per)
    q, r = divmod(T, 8)
    runs = []
    for x in range(8):
        b0 = x * q + min(x, r)
        b1 = b0 + q + (1 if x < r else 0)
        runs.append((b0 * per, min(b1 * per, n)))
    return runs


@pytest.mark.parametrize("case", ["gemv", "fused", "skinny", "base3", "split"])
def test_plan_unit_order(case):
    torch = torch_cuda()
    L = bl()
    big = [(28672, 2048), (8192, 8192), (1024, 4096), (8192, 8192)] * 12   # 8640 64-row groups
    small = [(3200, 3200), (3200, 8640), (1024, 3200), (8640, 3200)]
    fmt2, fmt3 = L.BITLINEAR_FORMAT_2BIT, L.BITLINEAR_FORMAT_BASE3
    shapes, M, fmt, kernel = {"gemv": (big, 1, fmt2, 0), "fused": (small, 1, fmt2, 7),
                              "skinny": (big, 16, fmt2, 2), "base3": (big, 1, fmt3, 8),
                              "split": (small + [(256, 20480)], 3, fmt2, 6)}[case]
    plan, units = _plan_units(L, torch, shapes, M, fmt)
    assert plan.kernel == kernel
    if fmt == fmt3:
        per_unit = 4                                            # 256-row blocks per unit at one token
        nu = [-(-(-(-N // 256)) // per_unit) for N, _ in shapes]

        def length(u):
            N, K = shapes[u[0]]
            blocks = min(per_unit, -(-N // 256) - u[1] * per_unit)
            return -(-K // 80) * blocks
    else:
        rows = 256 if kernel == 2 else 64
        nu = [-(-N // rows) for N, _ in shapes]

        def length(u):
            return -(-shapes[u[0]][1] // 64)
    if case == "split":
        # problem-major, blocks in order, a block's slices adjacent
        seen = [(p, g) for p, g in units]
        assert seen == sorted(seen)
        assert sorted(set(seen)) == [(p, g) for p in range(len(shapes)) for g in range(nu[p])]
        assert len(units) > sum(nu)
        return
    assert sorted(units) == [(p, g) for p in range(len(shapes)) for g in range(nu[p])]
    runs = [(0, len(units))] if case == "fused" else _xcd_runs(len(units), 4 if case == "gemv" else 1)
    for u0, u1 in runs:
        run = units[u0:u1]
        lens = [length(u) for u in run]
        assert lens == sorted(lens, reverse=True)
        # stable: equal lengths keep the table's problem, unit order
        for a, b in zip(run, run[1:]):
            if length(a) == length(b):
                assert a < b


@pytest.mark.parametrize("M", [2, 6, 8, 24])
def test_grouped_near_tie_rows(M):
    # The grouped quantizer (and the fused decode's own quantization at M <= 4)
    # on rows whose quotients x * 127 / eta sit on and next to rounding ties
    # (scaling a row by a power of two keeps every quotient): x~, eta and y
    # bit for bit against the oracle.
    torch = torch_cuda()
    L = bl()
    base = near_tie_rows()                                   # 6 rows, K = 3792
    K = base.shape[1]
    rows = np.concatenate([base * np.float32(sign * 2.0 ** e) for e in (0, 1, -1, 3) for sign in (1, -1)])
    specs, refs = [], []
    for i, N in enumerate((320, 1088)):
        x_np = np.ascontiguousarray(rows[i * M:(i + 1) * M])
        W = S.random_latent(900 + i, N, K)
        packed, g = pack_weights(W)
        Wt, _ = oracle.quantize_weights(W)
        specs.append(dict(x=torch.from_numpy(x_np).cuda(), xq=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                          eta=torch.empty(M, dtype=torch.float32, device="cuda"), packed=packed,
                          y=torch.empty((M, N), dtype=torch.float32, device="cuda"),
                          y_int=torch.empty((M, N), dtype=torch.int32, device="cuda"), gamma=g, N=N, K=K))
        refs.append((x_np, Wt, g))
    probs = L.make_problems(specs)
    tb = L.bitlinear_grouped_table_bytes(probs, len(specs), M)
    table = torch.empty(tb, dtype=torch.uint8, device="cuda")
    plan = L.bitlinear_grouped_plan_init(probs, len(specs), M, table, tb)
    say(f"grouped near-tie rows M={M} kernel={plan.kernel} quant_rows={plan.quant_rows}")
    L.bitlinear_forward_grouped(plan)
    torch.cuda.synchronize()
    for s, (x_np, Wt, g) in zip(specs, refs):
        y_ref, xq_ref, eta_ref, y_int_ref = oracle.forward(x_np, Wt, g, threads=THREADS)
        assert np.array_equal(s["xq"].cpu().numpy(), xq_ref)
        assert np.array_equal(s["eta"].cpu().numpy().view(np.uint32), eta_ref.view(np.uint32))
        assert np.array_equal(s["y_int"].cpu().numpy(), y_int_ref)
        assert np.array_equal(s["y"].cpu().numpy().view(np.uint32), y_ref.view(np.uint32))
