"""Host logic of bench.py that needs no GPU: launch classification and the
power/clock summary (with a stand-in for the driver's GPU metrics)."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_classify_gram_and_nxn():
    names = {1: "gns::transpose_sumsq<...>", 2: "gns::norm_finish(...)",
             3: "void gns::gemm_nt<gns::EBF16, 256, 0, 1, 0, 0>(gns::GemmParams)",
             4: "void gns::gemm_nt<gns::EBF16, 256, 0, 1, 0, 0>(gns::GemmParams)",
             5: "void gns::gemm_nt<gns::EBF16, 256, 1, 1, 1, 0>(gns::GemmParams)",
             6: "void gns::gemm_nt<gns::EBF16, 256, 0, 1, 0, 0>(gns::GemmParams)",
             7: "void gns::gemm_nt<gns::EBF16, 256, 0, 1, 0, 0>(gns::GemmParams)"}
    k = bench.classify(names)
    assert k[3] == "gemm_nt<bf16,256,sym>:gram"     # first symmetric launch after the norm
    assert k[4] == "gemm_nt<bf16,256,sym>:nxn"
    assert k[5] == "gemm_nn<bf16,256,gen>"
    assert k[6] == "gemm_nt<bf16,256,sym>:gram"     # after a general product (a restart)
    assert k[7] == "gemm_nt<bf16,256,sym>:nxn"


class _FakeSmi:
    """Stands in for the amdsmi module: a metrics table that refreshes every
    second call (about 1400 W: 1400 J per second in 2^-16 J units, 1000
    accumulation ticks per second, 995 of them throttled) and a power cap."""
    def __init__(self):
        self.calls = 0

    def amdsmi_get_gpu_metrics_info(self, h):
        self.calls += 1
        k = self.calls // 2                                   # table index
        return {"firmware_timestamp": 10 ** 8 * k, "energy_accumulator": int(1400 * 65536) * k,
                "accumulation_counter": 1000 * k, "ppt_residency_acc": 995 * k,
                "current_gfxclks": [1600 + k, 1700 + k, "N/A", 65535]}

    def amdsmi_get_power_cap_info(self, h):
        return {"power_cap": 1400 * 10 ** 6}


def _sampler(fake):
    s = bench.SmiSampler.__new__(bench.SmiSampler)
    s.period, s.tables, s.h, s.smi, s._thread = 0.0, [], object(), fake, None
    return s


def test_smi_window_summary_with_stand_in_metrics():
    s = _sampler(_FakeSmi())
    for _ in range(9):                                    # calls 1..9 -> tables 0..4 (each kept once)
        s._keep(s._metrics())
    assert len(s.tables) == 5
    out = s.summary()
    assert out["tables"] == 4                             # the table current at the start is dropped
    assert abs(out["socket_power_w"] - 1400.0) < 0.1
    assert out["ppt_residency_frac"] == 0.995
    assert out["power_cap_w"] == 1400.0                   # microwatts -> watts
    # clocks of tables 2..4 (the first table of the window may predate the load)
    assert out["gfxclk_mhz_min"] == 1602.0 and out["gfxclk_mhz_max"] == 1704.0
    assert out["gfxclk_mhz_mean"] == 1653.0


def test_smi_too_few_tables_or_absent_gives_none():
    s = _sampler(_FakeSmi())
    s._keep(s._metrics()); s._keep(s._metrics()); s._keep(s._metrics())   # tables 0, 1
    assert s.summary() is None
    t = _sampler(None)
    assert t.summary() is None
