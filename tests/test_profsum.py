"""The rocprofv3 summary writer: copy-probe scaling of the HBM byte counters,
the fp32 MFMA flop and busy-cycle figures, and the source-hash gate through
which bench.py reads them (host logic, synthetic CSVs in rocprofv3's format)."""
import csv
import os

from two_sided_gptq_amd import profsum

BAND = "bakron::(anonymous namespace)::band_gemm_kernel(bakron::(anonymous namespace)::BandArgs)"
COPY = "__amd_rocclr_copyBuffer"
QP = "bakron::(anonymous namespace)::qparams_kernel(int)"
FIN = "bakron::(anonymous namespace)::sumsq_final_kernel(int)"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def _counters(path, entries):
    # entries: (kernel, counter, value)
    _write(path, ["Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"],
           [[k, c, v, 0, 1] for k, c, v in entries])


def _fixture(tmp_path):
    tr = str(tmp_path / "trace")
    t, rows = 1000, []
    for name, dur in [(QP, 5000), (BAND, 20000), (BAND, 30000), (QP, 5000), (BAND, 25000), (FIN, 1000)]:
        rows.append([name, t, t + dur])
        t += dur + 100
    _write(os.path.join(tr, "bench_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    _write(os.path.join(tr, "bench_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "Percentage"],
           [[BAND, 3, 25000.0, 90.0], [QP, 2, 5000.0, 8.0]])
    pm = str(tmp_path / "pmc")
    # the 1 GiB copy shows FETCH_SIZE 512 MiB and WRITE_SIZE 1 GiB (in KiB):
    # scales x2 and x1
    _counters(os.path.join(pm, "FETCH_SIZE", "run_counter_collection.csv"),
              [(COPY, "FETCH_SIZE", 524288.0), (BAND, "FETCH_SIZE", 100.0), (BAND, "FETCH_SIZE", 300.0)])
    _counters(os.path.join(pm, "WRITE_SIZE", "run_counter_collection.csv"),
              [(COPY, "WRITE_SIZE", 1048576.0), (BAND, "WRITE_SIZE", 50.0), (BAND, "WRITE_SIZE", 50.0)])
    # two dispatches of 2**30 and 3 * 2**30 fp32 MFMA flops (MOPS in units of 512)
    mops = [2 ** 21, 3 * 2 ** 21]
    ent = []
    for v in mops:
        ent += [(BAND, "SQ_INSTS_VALU_MFMA_MOPS_F32", float(v)),
                (BAND, "SQ_VALU_MFMA_BUSY_CYCLES", v * 512 / 64.0),
                (BAND, "GRBM_GUI_ACTIVE", 1e6)]
    ent += [(QP, "SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0), (QP, "SQ_VALU_MFMA_BUSY_CYCLES", 0.0)]
    _counters(os.path.join(pm, "MFMA", "run_counter_collection.csv"), ent)
    _counters(os.path.join(pm, "MfmaUtil", "run_counter_collection.csv"),
              [(BAND, "MfmaUtil", 10.0), (BAND, "MfmaUtil", 20.0)])
    return tr, pm


def test_summary_figures(tmp_path):
    tr, pm = _fixture(tmp_path)
    text = profsum.summarise(tr, pm, "trace cmd", "pmc cmd", "mfma cmd")
    md = str(tmp_path / "p.md")
    open(md, "w").write(text)
    # bytes: mean fetch 200 KiB x2 + mean write 50 KiB x1 = 450 KiB
    assert profsum.read_traffic(md, "band_gemm_kernel") == 450 * 1024
    # flops: mean of 2**30 and 3 * 2**30
    assert profsum.read_figure(md, "mfma_flops_per_dispatch", "band_gemm_kernel") == float(f"{2 ** 31:.6g}")
    assert profsum.read_figure(md, "mfma_flops_per_dispatch", "qparams_kernel") is None
    # busy share: 2**31 / 64 busy cycles over 1024 SIMDs x 25 us x 2.4 GHz
    share = 2 ** 31 / 64 / (1024 * 25e-6 * 2.4e9)
    row = next(line for line in text.splitlines() if line.startswith("| band_gemm_kernel | 2 |")
               and "64.0" in line)
    assert f"{share:.3f}" in row and "| 15.0 |" in row
    # the graph window (between the two parameter kernels) holds the first two band launches
    assert "| band_gemm_kernel | 2 | 50.0 | 25.00 | 20.00 | 30.00 |" in text


def test_figures_gated_by_source_hash(tmp_path):
    tr, pm = _fixture(tmp_path)
    text = profsum.summarise(tr, pm, "t", "p", "m")
    md = str(tmp_path / "p.md")
    open(md, "w").write(text.replace(profsum.source_hash(), "0" * 16))
    assert profsum.read_traffic(md, "band_gemm_kernel") is None
    assert profsum.read_figure(md, "mfma_flops_per_dispatch", "band_gemm_kernel") is None
    assert profsum.read_traffic(str(tmp_path / "missing.md"), "band_gemm_kernel") is None


def test_summary_without_mfma_pass(tmp_path):
    tr, pm = _fixture(tmp_path)
    import shutil
    shutil.rmtree(os.path.join(pm, "MFMA"))
    text = profsum.summarise(tr, pm, "t", "p", "m")
    assert "MFMA work" not in text and "mfma_flops_per_dispatch" not in text
    assert "traffic_bytes_per_dispatch: band_gemm_kernel" in text



def test_windows_split_setup():
    """Solves are told apart by their final reductions: a solve with a side
    stream launches its parameter kernel twice, the second time among its first
    leaves and band launches."""
    LEAF = "bakron::(anonymous namespace)::leaf_kernel<false>(bakron::(anonymous namespace)::LeafArgs, int, int)"
    seq = [BAND,                                   # an earlier call
           QP, BAND, QP, LEAF, BAND, FIN,          # a graph solve
           QP, BAND, QP, LEAF, FIN,                # the timed graph solve
           COPY, QP, LEAF, BAND, FIN,              # the timing pass
           BAND, BAND]                             # band replays
    rows, t = [], 0
    for name in seq:
        rows.append({"Kernel_Name": name, "Start_Timestamp": str(t), "End_Timestamp": str(t + 10)})
        t += 20
    g, tp, rp = profsum._windows(rows)
    assert [r["Kernel_Name"] for r in g] == [QP, BAND, QP, LEAF, FIN]
    assert [r["Kernel_Name"] for r in tp] == [QP, LEAF, BAND, FIN]
    assert [r["Kernel_Name"] for r in rp] == [BAND, BAND]
