"""Host-side pieces of bench.py: kernel names from rocprofv3 symbols (both
the demangled and the mangled forms), the per-launch work model, the --gpus
guard.  No GPU."""
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402
import workloads  # noqa: E402

NS = "favor::(anonymous namespace)::"


@pytest.mark.parametrize("sym,short", [
    (f"void {NS}kpart<64, 4, 2, false>(unsigned short const*)", "kpart"),
    (f"void {NS}cscan<4, false, false>(unsigned short const*)", "cscan"),
    (f"void {NS}cscan<4, true, true>(unsigned short const*)", "cscan_lp"),
    (f"void {NS}bqr<256, false, 0>(unsigned short const*)", "bq_den"),
    (f"void {NS}bqr<256, true, 2>(unsigned short const*)", "bq_g"),
    (f"void {NS}bkeyr<128, false, 1>(unsigned short const*)", "bkey_dv"),
    (f"void {NS}cbk<8, false, 0, 2>(unsigned short const*)", "cbk_dk"),
    (f"void {NS}cbk<4, true, 1, 4>(unsigned short const*)", "cbk_dv"),
    (f"void {NS}cbq<8, false, 2>(unsigned short const*)", "cbq"),
    (f"{NS}cbsuffix(float*, float const*, float const*, int, int, int)", "cbsuffix"),
    ("_ZN5favor12_GLOBAL__N_15kpartILi64ELi4ELi2ELb0EEEvPKtS3_", "kpart"),
    ("_ZN5favor12_GLOBAL__N_15cscanILi4ELb1ELb0EEEvPKtS3_", "cscan"),
    ("_ZN5favor12_GLOBAL__N_15cscanILi4ELb0ELb1EEEvPKtS3_", "cscan_lp"),
    ("_ZN5favor12_GLOBAL__N_13bqrILi256ELb0ELi1EEEvPKt", "bq_dq"),
    ("_ZN5favor12_GLOBAL__N_13cbkILi8ELb0ELi0ELi2EEEvPKt", "cbk_dk"),
    ("_ZN5favor12_GLOBAL__N_13cbkILi4ELb0ELi1ELi4EEEvPKt", "cbk_dv"),
    ("void at::native::vectorized_elementwise_kernel<4>(int)", None),
])
def test_kernel_names_from_symbols(sym, short):
    assert bench._favor_kernel(sym) == short


def test_backward_work_model_sums_to_the_pass_totals():
    # Bytes: the causal matrix-core backward moves 7 d elements per
    # token*head once (kpart: K, V; the (L, p) scan: Q, dO; dq, dk, dv
    # writes), like the bidirectional passes.
    w = workloads.workload("text_causal").with_(causal=True)
    th = w.heads * w.L
    names = ("cscan_lp", "cbq", "cbg", "cbk_dk", "cbk_dv")
    nbytes = sum(bench.kernel_work(n, w, 1, w.L, 2)[0] for n in names)
    nbytes += bench.kernel_work("kpart", w, 1, w.L, 2, backward=True)[0]   # K and V
    assert nbytes == 7 * w.d * 2 * th
    wb = workloads.workload("text_bidir")
    names = ("bq_den", "bq_dq", "bq_g", "bkey_dk", "bkey_dv")
    nbytes = sum(bench.kernel_work(n, wb, 1, wb.L, 2)[0] for n in names)
    assert nbytes + 2 * wb.d * 2 * wb.heads * wb.L == 7 * wb.d * 2 * wb.heads * wb.L


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


@pytest.mark.parametrize("name,causal", [("text_bidir", False), ("text_causal", True),
                                         ("protein_long", True), ("wide_many", False)])
def test_forward_work_model_sums_to_the_call_totals(name, causal):
    # Each forward call moves 4 d elements per token*head once and does
    # 8 d m flops; the per-kernel figures add up to exactly that (a causal
    # segment-state pass that re-reads K and V is credited nothing).
    w = workloads.workload(name).with_(causal=causal)
    th = w.heads * w.L
    names = (("ckey", "kprefix", "cscan") if causal else ("kpart", "kcombine", "qapply"))
    if name == "wide_many":
        names = ("kpart", "kcombine", "qstream")
    if name == "text_bidir":
        names = ("fprep", "fused")   # the persistent kernel (64 heads, d 64, m 256)
    nb = sum(bench.kernel_work(n, w, 8, 512, 2)[0] for n in names)
    nf = sum(bench.kernel_work(n, w, 8, 512, 2)[1] for n in names)
    assert nb == 4 * w.d * 2 * th
    assert nf == 8.0 * w.d * w.m * th
