"""Host logic of bench.py that needs no GPU: algorithmic bytes, the mapping
of profiled kernel names to the step's phases, and the turning of two
rocprofv3 --pmc runs into bytes per launch calibrated on the probes."""
import csv
import json

import pytest

import bench
import ep_inputs


def test_algorithmic_bytes_large16k():
    # 16384 tokens, hidden 7168, top-8, 16 ranks: worked by hand
    b = bench.algorithmic_bytes(ep_inputs.WORKLOADS["large16k"])
    T, H, K, R = 16384, 7168, 8, 16
    assert b["layout"] == 8 * T * K + T * R == 1_310_720
    assert b["dispatch"] == 2 * T * H + 2 * T * K * H + 16 * T * K == 2_116_026_368
    assert b["combine"] == 2 * T * K * H + 2 * T * H + 8 * T * K == 2_114_977_792


def test_algorithmic_bytes_fp8_rows():
    b = bench.algorithmic_bytes(ep_inputs.WORKLOADS["prefill4k"], fp8=True)
    row = 7168 + 4 * 56
    assert b["dispatch"] == 4096 * row * 9 + 16 * 4096 * 8


@pytest.mark.parametrize("name,one_call,family", [
    ("void epget::(anonymous namespace)::combine_kernel<8>(epget::CopyParams, unsigned short const*)", True,
     "combine"),
    ("void epget::(anonymous namespace)::dispatch_chunks_kernel<7, 2>(epget::LayoutParams, epget::CopyParams)",
     True, "layout_dispatch"),
    ("void epget::(anonymous namespace)::layout_dispatch_kernel<1, 1024>(epget::LayoutParams)", True,
     "layout_dispatch"),
    ("epget::(anonymous namespace)::layout_count_kernel(epget::LayoutParams)", True, "layout_dispatch"),
    ("epget::(anonymous namespace)::layout_count_kernel(epget::LayoutParams)", False, "layout"),
    ("void epget::(anonymous namespace)::layout_assign_kernel<16, 2>(epget::LayoutParams)", False, "layout"),
    ("void epget::(anonymous namespace)::dispatch_kernel<7, 128>(epget::CopyParams, epget::DispatchArgs)",
     False, "dispatch"),
    ("void (anonymous namespace)::read_kernel<false>(unsigned int __vector(4) const*, long)", True, "probe_read"),
    ("void (anonymous namespace)::write_kernel<true>(unsigned int __vector(4)*, long)", True, "probe_write"),
    ("__amd_rocclr_copyBuffer", True, None),
    ("void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<unsigned char> >", True, None),
])
def test_kernel_families(name, one_call, family):
    assert bench._kernel_family(name, one_call) == family


def _pmc_csv(path, counter, rows):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for d, (name, value) in enumerate(rows):
            # each dispatch reported as two instances, summed by the reader
            for part in (0.25, 0.75):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": value * part})


def test_write_traffic_calibrates_on_probes(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    gib = 1 << 30
    count = "epget::(anonymous namespace)::layout_count_kernel(epget::LayoutParams)"
    disp = "void epget::(anonymous namespace)::dispatch_chunks_kernel<7, 2>(epget::LayoutParams)"
    comb = "void epget::(anonymous namespace)::combine_kernel<8>(epget::CopyParams)"
    rd = "void (anonymous namespace)::read_kernel<false>(unsigned int __vector(4) const*, long)"
    wr = "void (anonymous namespace)::write_kernel<false>(unsigned int __vector(4)*, long)"
    # the read counter sees half the bytes (factor 2), the write counter all
    fetch = [(count, 100.0), (disp, 1000.0), (comb, 8000.0)] * 3 + [(rd, gib / 2 / 1024), (wr, 0.0)]
    write = [(count, 10.0), (disp, 9000.0), (comb, 1000.0)] * 3 + [(rd, 0.0), (wr, gib / 1024)]
    _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    rec = bench.write_traffic("large16k", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    assert rec["factor_fetch"] == pytest.approx(2.0) and rec["factor_write"] == pytest.approx(1.0)
    assert rec["steps"] == 3
    ld = rec["layout_dispatch"]
    assert ld["launches_per_step"] == 2
    assert ld["bytes_per_launch"] == pytest.approx((2 * 1100 + 9010) * 1024)
    assert rec["combine"]["bytes_per_launch"] == pytest.approx((2 * 8000 + 1000) * 1024)
    saved = json.load(open(tmp_path / "traffic.json"))
    assert "large16k" in saved["workloads"]
    # the record is used while the sources are unchanged
    assert bench.measured_traffic("large16k", "combine") == pytest.approx(17000 * 1024)


def test_probe_library_exports_and_refuses_bad_sizes():
    """libepprobe.so (the ceilings' probe kernels) loads, lists its gather and
    scatter shapes, and refuses bad sizes before launching anything."""
    import ctypes

    lib = bench.probe_lib()
    for name in ("ep_probe_read", "ep_probe_write", "ep_probe_copy", "ep_probe_mix", "ep_probe_mix_shapes",
                 "ep_probe_mix_shape", "ep_probe_empty"):
        assert hasattr(lib, name), name
    assert lib.ep_probe_mix_shapes(0) == 6 and lib.ep_probe_mix_shapes(1) == 7
    v, nt, w = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert lib.ep_probe_mix_shape(1, 4, ctypes.byref(v), ctypes.byref(nt), ctypes.byref(w)) == 0
    assert (v.value, nt.value, w.value) == (7, 128, 0)
    assert lib.ep_probe_mix_shape(0, 6, ctypes.byref(v), ctypes.byref(nt), ctypes.byref(w)) == -1
    fake = 1 << 20   # never dereferenced: the size checks come first
    assert lib.ep_probe_read(fake, 0, 0, fake, None) == -1
    assert lib.ep_probe_write(fake, 24, 0, None) == -1
    assert lib.ep_probe_copy(fake, fake + 8, 1 << 20, None) == -1    # misaligned
    assert lib.ep_probe_mix(0, 0, fake, fake, 8, None) == -1
