"""The C ABI library on the CPU: it loads without a GPU, exports every call
include/bitlinear.h declares, the header compiles as C and C++, host-only size
queries are right, and argument validation returns the documented status
before anything touches a device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))
CSRC = os.path.join(ROOT, "ternary_weight_linear_fwd_amd", "csrc")

bl = pytest.importorskip("ternary_weight_linear_fwd_amd.bitlinear",
                         reason="libbitlinear.so not built (run __graft_entry__.build())")


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(bitlinear_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(bl.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bl.EXPORTED)
    out = subprocess.check_output(["nm", "-D", "--defined-only", bl.LIB_PATH], text=True)
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported


@pytest.mark.parametrize("lang,compiler", [("c", "gcc"), ("c++", "g++")])
def test_header_compiles(lang, compiler, tmp_path):
    src = tmp_path / ("t." + ("c" if lang == "c" else "cpp"))
    src.write_text('#include "bitlinear.h"\n#include "bitlinear_measure.h"\n'
                   'int main(void){ bitlinear_problem p; (void)p; '
                   'return (int)sizeof(bitlinear_grouped_plan) > 0 ? 0 : 1; }\n')
    subprocess.check_call([compiler, "-std=c99" if lang == "c" else "-std=c++11", "-Wall",
                           "-Werror", "-pedantic", "-I", os.path.dirname(HEADER), "-fsyntax-only",
                           str(src)])


def test_struct_layouts_match_header():
    assert ctypes.sizeof(bl.BitLinearProblem) == 64
    assert ctypes.sizeof(bl.BitLinearGroupedPlan) == 48


def test_status_strings():
    assert bl.bitlinear_status_string(0) == "BITLINEAR_OK"
    for code in (-1, -2, -3, -4, -5):
        assert bl.bitlinear_status_string(code).startswith("BITLINEAR_E")
    assert bl.bitlinear_status_string(7) == "BITLINEAR_UNKNOWN"
    assert bl.bitlinear_abi_version() == 10200


def test_packed3_and_lut_workspace_bytes():
    assert bl.bitlinear_packed3_bytes(1, 16) == 1024
    assert bl.bitlinear_packed3_bytes(64, 80) == 1024
    assert bl.bitlinear_packed3_bytes(65, 96) == 4 * 1024
    assert bl.bitlinear_packed3_bytes(8192, 8240) == 8192 * 8240 // 5    # 1.6 bits per weight
    assert bl.bitlinear_packed3_bytes(0, 16) == 0 and bl.bitlinear_packed3_bytes(8, 20) == 0
    assert bl.bitlinear_lut_workspace_bytes(1, 64, 64, 2) == 0
    assert bl.bitlinear_lut_workspace_bytes(1, 8192, 8192, 1) % 256 == 0


def test_packed_bytes():
    assert bl.bitlinear_packed_bytes(64, 64) == 1024
    assert bl.bitlinear_packed_bytes(2048, 2048) == 2048 * 2048 // 4
    assert bl.bitlinear_packed_bytes(8640, 3200) == 8640 * 3200 // 4
    assert bl.bitlinear_packed_bytes(1, 16) == 1024          # one padded block
    assert bl.bitlinear_packed_bytes(65, 80) == 2 * 2 * 1024
    assert bl.bitlinear_packed_bytes(8, 15) == 0              # K % 16 != 0
    assert bl.bitlinear_packed_bytes(0, 64) == 0
    assert bl.bitlinear_packed_bytes(1 << 20, 1 << 20) == 0   # N*K >= 2^40


def test_workspace_bytes():
    for M, N, K in ((1, 2048, 2048), (8, 3200, 8640), (2048, 8640, 3200), (0, 64, 64)):
        ws = bl.bitlinear_workspace_bytes(M, N, K)
        assert ws >= M * K + 4 * M and ws % 256 == 0 and ws >= 2048
    # prefill sizes: xq, eta and the row sums, each 256-byte aligned
    assert bl.bitlinear_workspace_bytes(2048, 8640, 3200) >= 2048 * 3200 + 2 * 4 * 2048
    assert bl.bitlinear_workspace_bytes(-1, 64, 64) == 0


FAKE = 1 << 20  # an aligned non-null address; never dereferenced by a rejected call


def _rc(fn, *args):
    return getattr(bl._lib, fn)(*args)


def test_validation_before_any_device_work():
    L = bl
    # quantize: null pointers, bad sizes, misalignment
    assert _rc("bitlinear_quantize_act", None, 1, 64, FAKE, FAKE, None, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_quantize_act", FAKE, -1, 64, FAKE, FAKE, None, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_quantize_act", FAKE, 1, 24, FAKE, FAKE, None, None) == L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_quantize_act", FAKE + 4, 1, 64, FAKE, FAKE, None, None) == L.BITLINEAR_EINVAL
    # pack: workspace required
    assert _rc("bitlinear_pack_weights", FAKE, 64, 64, FAKE, None, None, None, 0, None) == L.BITLINEAR_EWORKSPACE
    assert _rc("bitlinear_pack_weights", FAKE, 64, 64, FAKE, None, None, FAKE, 16, None) == L.BITLINEAR_EWORKSPACE
    assert _rc("bitlinear_pack_weights", FAKE, 64, 0, FAKE, None, None, FAKE, 1 << 16, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_pack_ternary", None, 64, 64, FAKE, None, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_unpack_weights", FAKE, 64, 20, FAKE, None, None) == L.BITLINEAR_EUNSUPPORTED
    # forward: null output, bad K, split-K workspace missing
    assert _rc("bitlinear_forward", FAKE, FAKE, FAKE, ctypes.c_float(1.0), 1, 64, 64, None, None, None, 0, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_forward", FAKE, FAKE, FAKE, ctypes.c_float(1.0), 1, 64, 48 + 1, FAKE, None, None, 0, None) == L.BITLINEAR_EUNSUPPORTED
    need = L.bitlinear_workspace_bytes(1, 8192, 28672)   # a long K loop: split over workgroups
    assert need > 0
    assert _rc("bitlinear_forward", FAKE, FAKE, FAKE, ctypes.c_float(1.0), 1, 8192, 28672, FAKE, None, None, 0, None) == L.BITLINEAR_EWORKSPACE
    # prefill sizes: the row sums need the workspace
    assert _rc("bitlinear_forward", FAKE, FAKE, FAKE, ctypes.c_float(1.0), 128, 64, 64, FAKE, None, None, 0, None) == L.BITLINEAR_EWORKSPACE
    assert _rc("bitlinear_forward", FAKE, FAKE, FAKE, ctypes.c_float(1.0), 128, 64, 64, FAKE, None, FAKE, 256, None) == L.BITLINEAR_EWORKSPACE
    # measurement probes
    assert L.bitlinear_measure_sink_bytes() >= 4 * 2048
    assert _rc("bitlinear_measure_stream_read", None, 1024, FAKE, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_measure_stream_read", FAKE, 1000, FAKE, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_measure_stream_read", FAKE + 8, 1024, FAKE, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_measure_mfma_i8", FAKE, FAKE, 0, FAKE, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_measure_mfma_i8", FAKE, None, 10, FAKE, None) == L.BITLINEAR_EINVAL
    assert L.bitlinear_measure_mfma_ops(0) == 0.0
    # forward with row sums: the sums are required; otherwise as bitlinear_forward
    assert _rc("bitlinear_forward_xsum", FAKE, FAKE, None, FAKE, ctypes.c_float(1.0), 128, 64, 64, FAKE, None, None, 0, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_forward_xsum", FAKE, FAKE, FAKE + 2, FAKE, ctypes.c_float(1.0), 128, 64, 64, FAKE, None, None, 0, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_forward_xsum", FAKE, FAKE, FAKE, FAKE, ctypes.c_float(1.0), 128, 64, 40, FAKE, None, None, 0, None) == L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_forward_xsum", FAKE, FAKE, FAKE, FAKE, ctypes.c_float(1.0), 1, 8192, 28672, FAKE, None, None, 0, None) == L.BITLINEAR_EWORKSPACE
    assert _rc("bitlinear_forward_f32", FAKE, FAKE, ctypes.c_float(1.0), 4, 64, 64, FAKE, None, 0, None) == L.BITLINEAR_EWORKSPACE
    assert _rc("bitlinear_forward_f32", FAKE, FAKE, ctypes.c_float(1.0), 4, 64, 64, FAKE, FAKE + 8, 1 << 20, None) == L.BITLINEAR_EWORKSPACE
    assert _rc("bitlinear_pack_weights_absmedian", FAKE, 64, 64, FAKE, None, None, FAKE, 4096, None) == L.BITLINEAR_EWORKSPACE
    assert _rc("bitlinear_pack_weights_absmedian", None, 64, 64, FAKE, None, None, FAKE, 1 << 20, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_pack_weights_absmedian", FAKE, 64, 24, FAKE, None, None, FAKE, 1 << 20, None) == L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_pack_ternary3", None, 64, 64, FAKE, None, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_pack_ternary3", FAKE, 64, 20, FAKE, None, None) == L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_unpack_weights3", FAKE, 64, 64, None, None, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_pack_weights3", FAKE, 64, 64, FAKE, None, None, None, 0, None) == L.BITLINEAR_EWORKSPACE
    assert _rc("bitlinear_forward_lut", FAKE, FAKE, FAKE, 2, ctypes.c_float(1.0), 1, 64, 64, FAKE, None, None, 0, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_forward_lut", FAKE, FAKE, FAKE, 1, ctypes.c_float(1.0), 1, 64, 72, FAKE, None, None, 0, None) == L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_forward_lut", FAKE, None, FAKE, 0, ctypes.c_float(1.0), 1, 64, 64, FAKE, None, None, 0, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_forward_lut", FAKE, FAKE, FAKE, 1, ctypes.c_float(1.0), 1, 8192, 28672, FAKE, None, None, 0, None) == L.BITLINEAR_EWORKSPACE
    assert _rc("bitlinear_rmsnorm_quantize_act", None, 1, 64, FAKE, FAKE, None, None, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_rmsnorm_quantize_act", FAKE, 1, 64, FAKE, None, None, None, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_rmsnorm_quantize_act", FAKE, 1, 40, FAKE, FAKE, None, None, None) == L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_rmsnorm_quantize_act", FAKE, 1, 64, FAKE + 2, FAKE, None, None, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_forward_rmsnorm_f32", FAKE, FAKE, ctypes.c_float(1.0), 4, 64, 64, FAKE, None, 0, None) == L.BITLINEAR_EWORKSPACE
    assert _rc("bitlinear_forward_rmsnorm_f32", FAKE, None, ctypes.c_float(1.0), 4, 64, 64, FAKE, FAKE, 1 << 20, None) == L.BITLINEAR_EINVAL


def test_k_limit():
    """K above BITLINEAR_MAX_K (2^21) is refused by every call before any device
    work: past it the dot4 path's scaled field sums and the prefill tiles'
    32-bit operand offsets would wrap."""
    L = bl
    big = L.BITLINEAR_MAX_K + 16
    assert L.bitlinear_packed_bytes(64, L.BITLINEAR_MAX_K) > 0
    assert L.bitlinear_packed_bytes(64, big) == 0
    assert L.bitlinear_workspace_bytes(1, 64, big) == 0
    assert L.bitlinear_packed3_bytes(64, big) == 0
    assert L.bitlinear_lut_workspace_bytes(1, 64, big, 0) == 0
    f1 = ctypes.c_float(1.0)
    assert _rc("bitlinear_quantize_act", FAKE, 1, big, FAKE, FAKE, None, None) == L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_forward", FAKE, FAKE, FAKE, f1, 1, 64, big, FAKE, None, FAKE, 1 << 30, None) == \
        L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_forward_xsum", FAKE, FAKE, FAKE, FAKE, f1, 128, 64, big, FAKE, None, FAKE, 1 << 30,
               None) == L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_forward_f32", FAKE, FAKE, f1, 4, 64, big, FAKE, FAKE, 1 << 30, None) == \
        L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_pack_weights", FAKE, 64, big, FAKE, None, None, FAKE, 1 << 20, None) == \
        L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_forward_lut", FAKE, FAKE, FAKE, 0, f1, 1, 64, big, FAKE, None, FAKE, 1 << 30, None) == \
        L.BITLINEAR_EUNSUPPORTED
    specs = [dict(x=None, xq=FAKE, eta=FAKE + 256, packed=FAKE, y=FAKE, gamma=0.5, N=128, K=big)]
    assert bl.bitlinear_grouped_table_bytes(bl.make_problems(specs), 1, 1) == 0


def test_noalloc_validation():
    """The allocation-free forward refuses, before any device work, sizes whose
    workspace exceeds its fixed device array, and the usual bad arguments."""
    L = bl
    f1 = ctypes.c_float(1.0)
    M, N, K = 4096, 1024, 1 << 20
    assert L.bitlinear_workspace_bytes(M, N, K) > L.BITLINEAR_NOALLOC_SCRATCH_BYTES
    assert _rc("bitlinear_forward_f32_noalloc", FAKE, FAKE, f1, M, N, K, FAKE, None) == L.BITLINEAR_EWORKSPACE
    assert _rc("bitlinear_forward_f32_noalloc", None, FAKE, f1, 4, 64, 64, FAKE, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_forward_f32_noalloc", FAKE, FAKE, f1, 4, 64, 64, None, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_forward_f32_noalloc", FAKE + 4, FAKE, f1, 4, 64, 64, FAKE, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_forward_f32_noalloc", FAKE, FAKE, f1, 4, 64, 40, FAKE, None) == L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_forward_f32_noalloc", FAKE, FAKE, f1, 0, 64, 64, FAKE, None) == L.BITLINEAR_OK


def test_forward3_validation_and_workspace():
    """The base-3 forward checks its arguments before any device work; its
    workspace holds the K-split partial sums ([S][M][N] int32) or nothing."""
    L = bl
    f1 = ctypes.c_float(1.0)
    assert _rc("bitlinear_forward3", FAKE, FAKE, FAKE, f1, 1, 64, 64, None, None, None, 0, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_forward3", FAKE + 4, FAKE, FAKE, f1, 1, 64, 64, FAKE, None, None, 0, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_forward3", FAKE, FAKE, FAKE + 8, f1, 1, 64, 64, FAKE, None, None, 0, None) == L.BITLINEAR_EINVAL
    assert _rc("bitlinear_forward3", FAKE, FAKE, FAKE, f1, 1, 64, 40, FAKE, None, None, 0, None) == L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_forward3", FAKE, FAKE, FAKE, f1, 1, 64, L.BITLINEAR_MAX_K + 16, FAKE, None, None, 0,
               None) == L.BITLINEAR_EUNSUPPORTED
    assert _rc("bitlinear_forward3", FAKE, FAKE, FAKE, f1, 0, 64, 64, FAKE, None, None, 0, None) == L.BITLINEAR_OK
    for M, N, K in ((1, 28672, 8192), (1, 8192, 28672), (8, 8192, 28672), (20, 3200, 8640)):
        need = L.bitlinear_forward3_workspace_bytes(M, N, K)
        assert need % 256 == 0 and need >= 2 * 4 * M * N          # at least two K-slices
        assert _rc("bitlinear_forward3", FAKE, FAKE, FAKE, f1, M, N, K, FAKE, None, FAKE, need - 256,
                   None) == L.BITLINEAR_EWORKSPACE
        assert _rc("bitlinear_forward3", FAKE, FAKE, FAKE, f1, M, N, K, FAKE, None, FAKE + 16, need,
                   None) == L.BITLINEAR_EWORKSPACE
    # one slice (no workspace) when K is short and N alone fills the chip
    assert L.bitlinear_forward3_workspace_bytes(1, 131072, 160) == 0
    assert L.bitlinear_forward3_workspace_bytes(1, 64, 40) == 0      # invalid sizes: 0


def test_grouped_planner_validation():
    def probs(n, **over):
        specs = []
        for i in range(n):
            s = dict(x=None, xq=FAKE + 4096 * i, eta=FAKE + 256, packed=FAKE, y=FAKE, gamma=0.5,
                     N=128, K=64)
            s.update(over)
            specs.append(s)
        return bl.make_problems(specs)

    ok = probs(3)
    assert bl.bitlinear_grouped_table_bytes(ok, 3, 1) > 0
    assert bl.bitlinear_grouped_table_bytes(ok, 0, 1) == 0
    assert bl.bitlinear_grouped_table_bytes(probs(2, K=40), 2, 1) == 0
    bad = probs(2)
    bad[1].format = 2                                    # no such layout
    assert bl.bitlinear_grouped_table_bytes(bad, 2, 1) == 0
    mixed = probs(2)
    mixed[1].format = bl.BITLINEAR_FORMAT_BASE3          # one layout per plan
    assert bl.bitlinear_grouped_table_bytes(mixed, 2, 1) == 0
    b3 = probs(2, format=bl.BITLINEAR_FORMAT_BASE3)
    assert bl.bitlinear_grouped_table_bytes(b3, 2, 8) > 0
    assert bl.bitlinear_grouped_table_bytes(b3, 2, 9) == 0   # base-3 plans: up to 8 tokens
    # one xq buffer fed from two different float32 sources
    clash = bl.make_problems([dict(x=FAKE, xq=FAKE, eta=FAKE, packed=FAKE, y=FAKE, gamma=1, N=64, K=64),
                              dict(x=FAKE + 4096, xq=FAKE, eta=FAKE, packed=FAKE, y=FAKE, gamma=1, N=64, K=64)])
    assert bl.bitlinear_grouped_table_bytes(clash, 2, 1) == 0
    plan = bl.BitLinearGroupedPlan()
    rc = bl._lib.bitlinear_grouped_plan_init(ok, 3, 1, None, 0, ctypes.byref(plan), None)
    assert rc == bl.BITLINEAR_EWORKSPACE


def test_library_never_allocates():
    for f in os.listdir(CSRC):
        text = open(os.path.join(CSRC, f)).read()
        for banned in ("hipMalloc", "hipFree", "hipHostMalloc", "malloc(", "new "):
            assert banned not in text, (f, banned)


def test_single_hip_runtime_in_process():
    # the library must bind to torch's HIP runtime, never load a second copy
    import re
    maps = open("/proc/self/maps").read()
    assert len(set(re.findall(r"\S*libamdhip64\S*", maps))) == 1


def test_no_undefined_library_symbols():
    # every kernel stub and helper of the library is defined in the .so
    out = subprocess.check_output(["nm", "-D", "--undefined-only", bl.LIB_PATH], text=True)
    assert not [l for l in out.splitlines() if "_ZN2bl" in l]


def test_grouped_planner_splits_only_small_plans():
    """Host logic of the grouped planner (no GPU: table sizes only).  A plan
    whose row blocks leave CUs idle (one transformer block) splits its long K
    loops and keeps int32 partial sums in the table, so the table grows by
    at least one partial row per work unit for each extra token; a whole
    model's plan, or a small one whose K loops are all short, keeps whole K
    loops and its table does not grow with M (no activations to quantize
    here, so no per-row entries either)."""
    def plan_bytes(shapes, M, copies=1):
        specs = [dict(x=None, xq=FAKE + 4096 * i, eta=FAKE + 256, packed=FAKE, y=FAKE, gamma=0.5, N=N, K=K)
                 for i, (N, K) in enumerate(shapes * copies)]
        n = bl.bitlinear_grouped_table_bytes(bl.make_problems(specs), len(specs), M)
        assert n > 0
        return n

    block = [(3200, 3200)] * 4 + [(8640, 3200)] * 2 + [(3200, 8640)]   # hidden 3200 / FFN 8640
    model = [(8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192), (28672, 8192), (28672, 8192),
             (8192, 28672)]
    groups64 = sum((N + 63) // 64 for N, _ in block)
    blocks256 = sum((N + 255) // 256 for N, _ in block)
    # fused dot4 GEMV (M <= 4): one unit per 64-row group, no partial sums
    assert plan_bytes(block, 2) == plan_bytes(block, 1)
    assert plan_bytes(block, 4) == plan_bytes(block, 3) == plan_bytes(block, 1)
    assert plan_bytes(model, 2, copies=80) == plan_bytes(model, 1, copies=80)
    assert plan_bytes(model, 4, copies=80) == plan_bytes(model, 3, copies=80)
    # K past the fused kernel's limit (16384): the dot4 GEMV splits K instead,
    # 64-row units with partial sums per token
    long_k = [(256, 20480), (128, 4096)]
    assert plan_bytes(long_k, 4) - plan_bytes(long_k, 3) >= (256 // 64 + 128 // 64) * 64 * 4
    # streaming MFMA kernel (5 .. 16 tokens): 256-row units
    assert plan_bytes(block, 9) - plan_bytes(block, 8) >= blocks256 * 256 * 4
    assert plan_bytes(model, 9, copies=80) == plan_bytes(model, 8, copies=80)
    # 64 x 256 prefill tiles (17 tokens and up): only the long down projection splits
    assert plan_bytes(block, 97) - plan_bytes(block, 96) >= 256 * 4 * ((3200 + 255) // 256)
    short = [(2000, 80), (1500, 208), (300, 1008)]
    assert plan_bytes(short, 97) == plan_bytes(short, 96)
