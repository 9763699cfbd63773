"""Host-side checks of the rocprofv3 summary helpers: the stream calibration
of FETCH_SIZE / WRITE_SIZE and the per-leg source digest that bench.py
requires before it reports a traffic figure."""

import csv
import os

from nvfp4_paged_decode_amd import profiling as P


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_counters_scale_by_streams_and_sum_legs(tmp_path):
    rd = "void (anonymous namespace)::read_kernel<8>(unsigned int __vector(4) const*, unsigned long, unsigned int*)"
    wr = "void (anonymous namespace)::write_kernel<4>(unsigned int __vector(4)*, unsigned long)"
    copy = "void copyBuffer(char*, char const*)"
    # the 1 MiB read stream reads 512 KiB on FETCH_SIZE (x2 scale), the 1 MiB
    # write stream 1024 KiB on WRITE_SIZE (x1); copies (which torch also
    # launches for its own clones) play no part
    _write_counters(tmp_path / "f", "FETCH_SIZE", [
        (rd, 512), (rd, 512), (wr, 3), (copy, 99999),
        ("kvfp4::(anonymous namespace)::quantize_kernel(kvfp4::Geom)", 100),
        ("void kvfp4::(anonymous namespace)::decode_gqa_mfma_kernel<2>(int)", 30),
        ("kvfp4::(anonymous namespace)::merge_balanced_kernel<true>(int)", 10)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [
        (rd, 0), (wr, 1024), (wr, 1024), (copy, 99999),
        ("kvfp4::(anonymous namespace)::quantize_kernel(kvfp4::Geom)", 50),
        ("void kvfp4::(anonymous namespace)::decode_gqa_mfma_kernel<2>(int)", 1),
        ("kvfp4::(anonymous namespace)::merge_balanced_kernel<true>(int)", 2)])
    lines = P.counters(str(tmp_path / "f"), str(tmp_path / "w"), 1 << 20, "wl")
    traffic = {}
    for l in lines:
        if l.startswith("traffic "):
            kv = dict(p.split("=", 1) for p in l.split()[1:])
            traffic[kv["leg"]] = kv
    assert int(traffic["quantize"]["read_bytes"]) == 100 * 1024 * 2
    assert int(traffic["quantize"]["written_bytes"]) == 50 * 1024
    assert int(traffic["decode"]["total_bytes"]) == (30 + 10) * 2048 + (1 + 2) * 1024
    assert traffic["decode"]["sources"] == P.source_digest("decode")
    path = tmp_path / "counters.txt"
    path.write_text("\n".join(lines) + "\n")
    assert P.read_traffic(str(path), "wl", "quantize") == 100 * 2048 + 50 * 1024
    assert P.read_traffic(str(path), "other", "quantize") is None
    # a figure taken on other sources is not reported
    path.write_text("\n".join(lines).replace(P.source_digest("quantize"), "0" * 64) + "\n")
    assert P.read_traffic(str(path), "wl", "quantize") is None


def test_leg_digests_cover_their_sources():
    for leg, names in P.LEG_SOURCES.items():
        for n in names:
            assert os.path.exists(os.path.join(P.CSRC, n)), (leg, n)
    assert P.source_digest("decode") != P.source_digest("quantize")
    assert P.source_digest("quantize") == P.source_digest("dequantize")


def test_every_step_kernel_has_its_leg():
    """Each kernel the benchmark's step launches maps to its leg (traffic
    lines and rooflines are read per leg)."""
    ns = "void kvfp4::(anonymous namespace)::"
    for name, leg in [("quantize_kernel(kvfp4::Geom)", "quantize"),
                      ("quantize_rounds_kernel(kvfp4::Geom)", "quantize"),
                      ("dequantize_kernel(kvfp4::Geom)", "dequantize"),
                      ("sort_pages_kernel(int const*)", "sort"),
                      ("decode_gqa_mfma_kernel<128, 2, 1>(kvfp4::DecodeArgs)", "decode"),
                      ("merge_balanced_kernel<true, 1, 128, 128>(kvfp4::DecodeArgs)", "decode")]:
        assert P.leg_of(P.short_name(ns + name)) == leg, name


def test_names_outside_the_library_namespace_are_kept():
    """The benchmark's stream yardsticks live in an anonymous namespace of
    their own: they keep their names and belong to no leg."""
    n = P.short_name("void (anonymous namespace)::read4_write1_kernel<8>(unsigned int const*)")
    assert n == "read4_write1_kernel<8>"
    assert P.leg_of(n) is None


def test_pmc_summary_fractions(tmp_path):
    """The pmc summary merges passes per kernel and derives its shares from
    the averaged counters (GRBM_GUI_ACTIVE is the sum over 8 XCDs)."""
    k = "void kvfp4::(anonymous namespace)::decode_mla_kernel<4, 2>(kvfp4::DecodeArgs)"
    a = tmp_path / "a"
    b = tmp_path / "b"
    for d, rows in ((a, [("SQ_WAVE_CYCLES", 1000), ("SQ_WAIT_ANY", 600),
                         ("SQ_ACTIVE_INST_ANY", 250), ("SQ_VALU_MFMA_BUSY_CYCLES", 4096),
                         ("GRBM_GUI_ACTIVE", 80)]),
                    (b, [("SQ_ACTIVE_INST_LDS", 200), ("SQ_LDS_BANK_CONFLICT", 50),
                         ("GRBM_GUI_ACTIVE", 80)])):
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for c, v in rows:
                w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})
    lines = P.pmc([str(a), str(b)])
    row = next(l for l in lines if l.startswith("decode_mla_kernel<4, 2>"))
    cols = row.split()
    # kernel name has a space: "decode_mla_kernel<4," "2>"
    wait, issue, valu, lds, mfma, bank = cols[3:9]
    assert float(wait) == 60.0 and float(issue) == 25.0 and valu == "-"
    assert float(lds) == 20.0 and float(mfma) == 40.0 and float(bank) == 25.0
