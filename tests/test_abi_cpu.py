"""CPU-side checks of the C ABI and the host logic: the library loads, exports
every function the header declares, rejects bad arguments before enqueuing
anything, and the planner's decompositions cover every output column and K
value exactly once.  No GPU is needed (plan creation does not touch HIP)."""
import json
import math
import os

import pytest

import chiplet_aware_persistent_amd as sg
from chiplet_aware_persistent_amd import model

GOLD = os.path.join(os.path.dirname(__file__), "golden")

pytestmark = pytest.mark.skipif(not os.path.exists(sg.LIB_PATH), reason="libsgemm.so not built")


def test_exports_every_header_function():
    names = sg.header_functions()
    assert len(names) >= 10
    lib = sg.library()
    for n in names:
        assert hasattr(lib, n), n


def _create(**kw):
    p = sg.Problem(kw.get("kind", sg.KIND_GEMM), kw.get("M", 1), kw.get("K", 64), kw.get("N", 64),
                   kw.get("out", sg.OUT_F32), kw.get("L", 0), kw.get("d", 0), kw.get("q", 0), kw.get("dff", 0),
                   kw.get("flags", 0), kw.get("tn", 0), kw.get("splitk", 0), kw.get("waves", 0),
                   kw.get("ksl", 0))
    rc, h, ws = sg.sgemm_plan_create(p)
    if h:
        sg.sgemm_plan_destroy(h)
    return rc


@pytest.mark.parametrize("kw,code", [
    (dict(M=0), sg.ERR_INVALID_ARG),
    (dict(M=65), sg.ERR_UNSUPPORTED),
    (dict(K=12), sg.ERR_INVALID_ARG),
    (dict(K=0), sg.ERR_INVALID_ARG),
    (dict(N=0), sg.ERR_INVALID_ARG),
    (dict(out=7), sg.ERR_INVALID_ARG),
    (dict(flags=sg.F_FORCE_DOT2 | sg.F_FORCE_MFMA), sg.ERR_INVALID_ARG),
    (dict(waves=3), sg.ERR_INVALID_ARG),
    (dict(splitk=65), sg.ERR_UNSUPPORTED),
    (dict(ksl=3), sg.ERR_INVALID_ARG),
    (dict(ksl=-1), sg.ERR_INVALID_ARG),
    (dict(M=4, ksl=2), sg.ERR_UNSUPPORTED),               # K slices are an MFMA-path option
    (dict(M=16, K=4096, N=4096, ksl=8), sg.OK),
    (dict(kind=9), sg.ERR_INVALID_ARG),
    (dict(K=1 << 20, N=1 << 12), sg.ERR_UNSUPPORTED),
    (dict(kind=sg.KIND_LAYERCHAIN, M=4, L=0, d=64, q=64, dff=64), sg.ERR_INVALID_ARG),
    (dict(kind=sg.KIND_LAYERCHAIN, M=4, L=2, d=60, q=64, dff=64), sg.ERR_INVALID_ARG),
    (dict(kind=sg.KIND_LAYERCHAIN, M=4, L=65, d=64, q=64, dff=64), sg.ERR_UNSUPPORTED),
    (dict(kind=sg.KIND_LAYERCHAIN, M=65, L=2, d=64, q=64, dff=64), sg.ERR_UNSUPPORTED),
    (dict(M=1, K=8, N=1), sg.OK),
    (dict(M=32, flags=sg.F_MTILE_ITEMS | sg.F_FORCE_DOT2), sg.ERR_INVALID_ARG),
    (dict(M=32, K=1024, N=1024, flags=sg.F_MTILE_ITEMS, ksl=2), sg.ERR_UNSUPPORTED),
    (dict(M=32, K=1024, N=1024, flags=sg.F_MTILE_ITEMS), sg.OK),
    (dict(kind=sg.KIND_LAYERCHAIN, M=32, L=2, d=64, q=64, dff=64, flags=sg.F_MTILE_ITEMS), sg.ERR_UNSUPPORTED),
    (dict(M=64, K=12288, N=4096), sg.OK),
])
def test_plan_create_validation(kw, code):
    assert _create(**kw) == code


def test_null_and_misaligned_arguments_rejected_before_launch():
    lib = sg.library()
    assert lib.sgemm_plan_create(None, 0, None, None) == sg.ERR_INVALID_ARG
    g = sg.Gemm(4, 256, 128)
    h = g.handle
    assert sg.sgemm_run(h, 0, 16, 16, 16) == sg.ERR_INVALID_ARG
    assert sg.sgemm_run(h, 16, 0, 16, 16) == sg.ERR_INVALID_ARG
    assert sg.sgemm_run(h, 16, 16, 16, 0) == sg.ERR_INVALID_ARG
    assert sg.sgemm_run(h, 18, 16, 16, 16) == sg.ERR_INVALID_ARG   # misaligned X
    assert sg.sgemm_run(h, 16, 24, 16, 16) == sg.ERR_INVALID_ARG   # misaligned W
    assert sg.sgemm_run(None, 16, 16, 16, 16) == sg.ERR_INVALID_ARG
    assert sg.layerchain_run(h, 16, [16], [16], [16], [16], 16, 0, 16) == sg.ERR_INVALID_ARG  # kind
    assert sg.sgemm_workspace_init(h, 0) == sg.ERR_INVALID_ARG
    assert lib.sgemm_topology_probe(None, 4, None) == sg.ERR_INVALID_ARG
    assert sg.status_string(sg.ERR_TIMEOUT) == "device wait timed out"


SHAPES = [(1, 1024, 1024), (1, 4096, 6144), (1, 4096, 4096), (1, 4096, 24576), (1, 12288, 4096),
          (8, 4096, 6144), (16, 4096, 4096), (32, 4096, 24576), (64, 12288, 4096), (1, 7168, 1536),
          (2, 7168, 4096), (16, 7168, 18432), (3, 520, 1000), (17, 776, 530), (5, 8, 17), (64, 8, 1)]


@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("splitk", [0, 3])
@pytest.mark.parametrize("flags", [0, sg.F_MTILE_ITEMS])
def test_planner_covers_every_column_and_k_once(M, K, N, splitk, flags):
    if flags and M < 16:
        return
    try:
        g = sg.Gemm(M, K, N, splitk=splitk, flags=flags)
    except sg.SgemmError as e:
        # a forced split count whose X window exceeds the LDS budget is refused
        assert splitk and e.code == sg.ERR_UNSUPPORTED
        return
    st = g.describe()["stage"]
    assert st["path"] == ("dot2" if M < 16 else "mfma")
    mt = st["mtiles"]
    assert mt == (math.ceil(M / 16) if flags else 1) and (mt == 1 or st["ta"] == 1)
    assert 16 * st["ta"] * mt >= M                     # m-tiles cover every row
    Nx, CB, NB, S, KS = st["Nx"], st["CB"], st["NB"], st["S"], st["KS"]
    ksl, kss = st["ksl"], st["kss"]
    assert st["wpi"] % ksl == 0 and CB == st["wpi"] // ksl * st["TN"] and st["waves"] % st["wpi"] == 0
    assert ksl == 1 or (st["path"] == "mfma" and st["wpi"] == st["waves"])  # one item stream per workgroup
    assert 8 * Nx >= N and 8 * (Nx - 16) < N          # per-XCD partition covers N, no spare XCD block
    assert NB * CB >= Nx                               # column blocks cover the XCD's columns
    assert S * KS >= K and (S - 1) * KS < K            # splits cover K, none empty
    assert ksl * kss >= KS and (ksl - 1) * kss < KS    # slices cover a split, none empty
    assert KS % 64 == 0 and st["items"] == NB * S * mt  # splits start on 128-byte lines
    kstep = 512 if st["path"] == "dot2" else 64
    assert ksl == 1 or kss % kstep == 0
    assert st["steps"] * kstep >= kss
    assert st["lds"] <= 160 * 1024
    # every k of a split is streamed by exactly one slice, and the LDS window
    # holds what the last slice reads including its padded steps
    for s in range(S):
        seen = []
        for q in range(ksl):
            k0 = s * KS + q * kss
            klim = min(min(K, (s + 1) * KS) - k0, kss)
            seen += list(range(k0, k0 + max(klim, 0)))
        assert seen == list(range(s * KS, min(K, (s + 1) * KS)))
    assert st["win"] >= (ksl - 1) * kss + st["steps"] * kstep
    if splitk:
        assert S == math.ceil(K / (math.ceil(math.ceil(K / splitk) / 64) * 64))
    # columns: every column owned by exactly one (xcd, block, wave, lane-column)
    owned = set()
    for x in range(8):
        for b in range(NB):
            for c in range(CB):
                col = x * Nx + b * CB + c
                if x * Nx + b * CB + c < min(N, (x + 1) * Nx) and b * CB + c < Nx:
                    assert col not in owned
                    owned.add(col)
    assert owned == set(range(N))


def test_chain_plan_and_buffers():
    c = sg.LayerChain(64, 36, 4096, 4096, 12288)
    d = c.describe()
    assert d["kind"] == "layerchain" and len(d["stages"]) == 4
    assert d["stages"][2]["paired"] == 1 and d["stages"][2]["N"] == 12288
    spans = []
    for l in (0, 17, 35):
        for w in range(4):
            rc, off, nb = sg.sgemm_chain_buffer(c.handle, l, w)
            assert rc == 0 and off + nb <= c.workspace_bytes and off % 16 == 0
            spans.append((off, off + nb))
    spans.sort()
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    assert sg.sgemm_chain_buffer(c.handle, 36, 0)[0] == sg.ERR_INVALID_ARG
    assert sg.sgemm_chain_buffer(c.handle, 0, 4)[0] == sg.ERR_INVALID_ARG


def test_chain_path_choice():
    """dot2 stages at M <= 2 (G weight rows per wave, gate_up holding G/2
    gate/up pairs), MFMA stages above; SGEMM_F_FORCE_DOT2 (M < 16) and
    SGEMM_F_FORCE_MFMA choose the path, and FORCE_DOT2 is refused at M >= 16."""
    def paths(M, flags=0):
        return [s["path"] for s in sg.LayerChain(M, 4, 4096, 4096, 12288, flags=flags).describe()["stages"]]
    for M, flags in ((1, 0), (2, 0), (3, sg.F_FORCE_DOT2), (8, sg.F_FORCE_DOT2), (15, sg.F_FORCE_DOT2)):
        st = sg.LayerChain(M, 4, 4096, 4096, 12288, flags=flags).describe()["stages"]
        assert [s["path"] for s in st] == ["dot2"] * 4, M
        g = st[0]["tb"]
        assert g in (2, 4) and all(s["tb"] == g for s in st) and g * M <= 64
        assert st[2]["paired"] == 1 and st[2]["TN"] == g // 2 and st[0]["TN"] == g
    for M in (3, 8, 15, 16, 17, 64):
        assert paths(M) == ["mfma"] * 4, M
    assert paths(1, sg.F_FORCE_MFMA) == ["mfma"] * 4
    with pytest.raises(sg.SgemmError):
        sg.LayerChain(16, 4, 4096, 4096, 12288, flags=sg.F_FORCE_DOT2)


def test_chain_scheduler_plan():
    """With SGEMM_F_SCHEDULER the stages are planned over 31 worker slots per
    XCD (slot 0 schedules); the grid stays 8 x 32.  The mode is a chain runtime:
    refused for a single GEMM and with the flat or poll-leader counters."""
    for M in (1, 16, 64):
        base = sg.LayerChain(M, 4, 4096, 4096, 12288).describe()
        sch = sg.LayerChain(M, 4, 4096, 4096, 12288, flags=sg.F_SCHEDULER).describe()
        assert sch["grid"] == base["grid"] == 256
        assert [s["slots"] for s in base["stages"]] == [32] * 4
        assert [s["slots"] for s in sch["stages"]] == [31] * 4
        assert [s["path"] for s in sch["stages"]] == [s["path"] for s in base["stages"]]
    for flags in (sg.F_SCHEDULER | sg.F_SYNC_FLAT, sg.F_SCHEDULER | sg.F_POLL_LEADER):
        with pytest.raises(sg.SgemmError):
            sg.LayerChain(16, 4, 4096, 4096, 12288, flags=flags)
    with pytest.raises(sg.SgemmError):
        sg.Gemm(16, 4096, 4096, flags=sg.F_SCHEDULER)


def test_eq1_matches_the_pages_table():
    g = json.load(open(os.path.join(GOLD, "eq1_l2_hit.json")))
    for row in g["rows"]:
        assert model.eq1_hit(row["B"], W=g["W"], T_M=g["T_M"]) == pytest.approx(row["predicted_hit"])
    assert model.eq1_hit(10 ** 6, W=g["W"]) == pytest.approx(g["limit_hit_W31"], abs=1e-4)
    ex = g["ai_eff_example"]
    assert model.ai_eff(ex["B"], ex["hit"]) == pytest.approx(ex["ai_eff_approx"], rel=0.02)


def test_roofline_floors():
    # 2*K*N bytes at 8 TB/s: QKV 4096x6144 -> 6.29 us, down 12288x4096 -> 12.58 us
    assert model.floor_us(4096, 6144) == pytest.approx(6.29, abs=0.01)
    assert model.floor_us(12288, 4096) == pytest.approx(12.58, abs=0.01)
    assert model.ridge_flop_per_byte() == pytest.approx(312.5)


def test_build_reads_scratch_usage_from_compiler_remarks():
    from chiplet_aware_persistent_amd import build
    remarks = "\n".join([
        "x.hip:14:1: remark: Function Name: _ZN2sg4k_aEv [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:14:1: remark:     VGPRs: 105 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:14:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:21:1: remark: Function Name: _ZN2sg4k_bEv [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:21:1: remark:     ScratchSize [bytes/lane]: 3136 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build.scratch_usage(remarks) == {"_ZN2sg4k_aEv": 0, "_ZN2sg4k_bEv": 3136}


def test_read_probe_rejects_bad_arguments_before_launch():
    lib = sg.library()
    assert lib.sgemm_read_probe(None, 1024, 0, 16, 256, None) == sg.ERR_INVALID_ARG
    assert lib.sgemm_read_probe(16, 1024, 0, None, 256, None) == sg.ERR_INVALID_ARG
    assert lib.sgemm_read_probe(24, 1024, 0, 16, 256, None) == sg.ERR_INVALID_ARG    # misaligned source
    assert lib.sgemm_read_probe(16, 1024, 0, 18, 256, None) == sg.ERR_INVALID_ARG    # misaligned sink
    assert lib.sgemm_read_probe(16, 1000, 0, 16, 256, None) == sg.ERR_INVALID_ARG    # not whole 16-byte chunks
    assert lib.sgemm_read_probe(16, 1 << 31, 0, 16, 256, None) == sg.ERR_INVALID_ARG  # past the buffer extent
    assert lib.sgemm_read_probe(16, 1024, 2, 16, 256, None) == sg.ERR_INVALID_ARG    # pattern
    assert lib.sgemm_read_probe(16, 1024, 0, 16, 12, None) == sg.ERR_INVALID_ARG     # grid not a multiple of 8
    assert lib.sgemm_read_probe(16, 1024, 0, 16, 8192, None) == sg.ERR_INVALID_ARG


@pytest.mark.parametrize("name,value,kind", [
    ("SGEMM_SPLITK", "two", sg.KIND_GEMM), ("SGEMM_WAVES", "6", sg.KIND_GEMM), ("SGEMM_KSLICES", "3", sg.KIND_GEMM),
    ("SGEMM_TN", "-1", sg.KIND_GEMM), ("SGEMM_WATCHDOG_S", "abc", sg.KIND_LAYERCHAIN),
    ("SGEMM_WATCHDOG_S", "0", sg.KIND_LAYERCHAIN), ("SGEMM_CHAIN_COST", "1.5,75", sg.KIND_LAYERCHAIN),
    ("SGEMM_CHAIN_COST", "0.5,75,0.5,0.05,0.25", sg.KIND_LAYERCHAIN), ("SGEMM_CHAIN_S", "1,2", sg.KIND_LAYERCHAIN)])
def test_malformed_environment_overrides_are_rejected(monkeypatch, name, value, kind):
    monkeypatch.setenv(name, value)
    if kind == sg.KIND_GEMM:
        assert _create(M=16, K=1024, N=1024) == sg.ERR_INVALID_ARG
    else:
        assert _create(kind=kind, M=4, L=2, d=256, q=128, dff=384) == sg.ERR_INVALID_ARG


def test_environment_overrides_apply(monkeypatch):
    monkeypatch.setenv("SGEMM_SPLITK", "4")
    monkeypatch.setenv("SGEMM_WATCHDOG_S", "2.5")
    assert sg.Gemm(16, 4096, 1024).describe()["stage"]["S"] == 4
    assert _create(kind=sg.KIND_LAYERCHAIN, M=4, L=2, d=256, q=128, dff=384) == sg.OK


@pytest.mark.parametrize("lang,compiler", [("c", "gcc"), ("c++", "g++")])
def test_header_is_plain_c_and_cpp(tmp_path, lang, compiler):
    """include/sgemm.h compiles on its own as C and as C++ (no HIP types)."""
    import shutil
    import subprocess

    if not shutil.which(compiler):
        pytest.skip(compiler + " not found")
    src = tmp_path / ("t." + ("c" if lang == "c" else "cpp"))
    src.write_text('#include "sgemm.h"\nint main(void) { return SGEMM_F_MTILE_ITEMS != 0 ? 0 : 1; }\n')
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    r = subprocess.run([compiler, "-std=c11" if lang == "c" else "-std=c++17", "-Wall", "-Werror", "-fsyntax-only",
                        "-I", inc, str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_python_constants_match_the_header(tmp_path):
    """Every SGEMM_* enumerator of include/sgemm.h has the same value in the
    binding (flags, status codes, kinds, output types)."""
    import re
    import shutil
    import subprocess

    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    header = open(os.path.join(inc, "sgemm.h")).read()
    names = sorted(set(re.findall(r"\b(SGEMM_(?:F|ERR|KIND|OUT)_[A-Z0-9_]+|SGEMM_OK)\s*=", header)))
    assert len(names) > 15
    src = tmp_path / "c.c"
    src.write_text('#include <stdio.h>\n#include "sgemm.h"\nint main(void) {\n' +
                   "".join('  printf("%s %%lld\\n", (long long)%s);\n' % (n, n) for n in names) + "  return 0;\n}\n")
    exe = tmp_path / "c"
    r = subprocess.run(["gcc", "-std=c11", "-I", inc, str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    for line in out.splitlines():
        name, value = line.split()
        py = name[len("SGEMM_"):]
        assert hasattr(sg, py), name
        assert getattr(sg, py) == int(value), (name, getattr(sg, py), value)


def test_chain_stamps_breakdown_on_a_made_up_timeline():
    """Two workgroups and five events (Q, O, gate_up and down of one layer,
    then Q of the next); every figure is worked out by hand below."""
    import numpy as np
    from chiplet_aware_persistent_amd.chain_stamps import stage_breakdown
    st = np.zeros((2, 5, 2))
    t = 0.0
    for e in range(5):
        st[0, e] = (t + 1.0, t + 5.0)   # workgroup 0 starts 1 us after the barrier, works 4 us
        st[1, e] = (t + 2.0, t + 8.0)   # workgroup 1 starts 2 us after, works 6 us
        t += 8.0
    b = stage_breakdown(st)
    assert set(b) == {"Q", "O", "gate_up", "down"}
    # release: first start (t+1) minus the previous last end (t)
    # skew 1; med_start 0.5; work_med 5; tail: 8 - median(5, 8) = 1.5; span: 8 - 1 = 7
    for v in b.values():
        assert v == [1.0, 1.0, 0.5, 5.0, 1.5, 7.0]


def test_bench_cpu_baselines_report_the_contract_fields():
    """Both workloads' CPU baselines time the oracle as it stands and say what
    they timed (tiny shapes here; the bench uses the full ones)."""
    import bench
    import synth
    x = synth.normal_bf16(1, 2, 256)
    ws = [synth.uniform_bf16(2, 128, 256, 0.05), synth.uniform_bf16(3, 256, 128, 0.05),
          synth.uniform_bf16(4, 2 * 384, 256, 0.05), synth.uniform_bf16(5, 256, 384, 0.05)]
    r = bench.cpu_baseline_chain(2, x, ws)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0 and r["cores"] >= 1
    assert "M=2" in r["sample"]
