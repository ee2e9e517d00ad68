"""Host logic of bench.py that runs without a GPU: the shader-clock sampler
(which SMU refreshes count, which device is read) and its behaviour when
amdsmi is missing."""
import sys
import time
import types

import bench


class _Props:
    pci_domain_id, pci_bus_id, pci_device_id = 0, 0x8B, 0


class _Cuda:
    def get_device_properties(self, i):
        return _Props()

    def synchronize(self):
        pass


class _Torch:
    cuda = _Cuda()


def _fake_amdsmi(refreshes, polls_per_refresh=2):
    """A stand-in for amdsmi whose metrics advance to the next refresh every
    `polls_per_refresh` polls (the last one stays); two devices, the second
    at cuda:0's PCI address."""
    m = types.ModuleType("amdsmi")
    state = {"polls": 0, "inited": 0, "shut": 0, "read": set()}

    def metrics(h):
        state["read"].add(h)
        i = min(state["polls"] // polls_per_refresh, len(refreshes) - 1)
        state["polls"] += 1
        return refreshes[i]

    m.amdsmi_init = lambda: state.__setitem__("inited", state["inited"] + 1)
    m.amdsmi_shut_down = lambda: state.__setitem__("shut", state["shut"] + 1)
    m.amdsmi_get_processor_handles = lambda: ["gpu_a", "gpu_b"]
    m.amdsmi_get_gpu_device_bdf = lambda h: "0000:8b:00.0" if h == "gpu_b" else "0000:05:00.0"
    m.amdsmi_get_gpu_metrics_info = metrics
    return m, state


def _refresh(acc, activity, clocks):
    return {"gfx_activity_acc": acc, "average_gfx_activity": activity, "current_gfxclks": clocks}


def test_sclk_counts_fresh_busy_refreshes_only(monkeypatch):
    refreshes = [
        _refresh(100, 0, [105, 106, 95, 95, 95, 95, 112, 112]),         # current when the calls start: dropped
        _refresh(200, 30, [1500] * 8),                                 # GPU under half busy: dropped
        _refresh(300, 100, [2000, 2000, 2000, 2000, 1900, 1900, 1900, 1900]),
        _refresh(300, 100, [1, 1, 1, 1, 1, 1, 1, 1]),                  # same accumulator: not a new refresh
        _refresh(400, 97, [2100, "N/A", 2100, 2100, 2100, 2100, 2100, 2100]),
    ]
    fake, state = _fake_amdsmi(refreshes)
    monkeypatch.setitem(sys.modules, "amdsmi", fake)
    calls = []
    r = bench.sclk_during(_Torch(), lambda: (calls.append(1), time.sleep(0.002)), seconds=0.4)
    assert state["read"] == {"gpu_b"}
    assert state["inited"] == 1 and state["shut"] == 1
    assert r["readings"] == 2, r
    assert r["mhz_min"] == 1950.0 and r["mhz_max"] == 2100.0
    assert r["mhz_median"] in (1950.0, 2100.0)
    assert r["calls"] == len(calls) > 0


def test_sclk_none_without_fresh_busy_readings(monkeypatch):
    fake, _ = _fake_amdsmi([_refresh(7, 100, [2000] * 8)])            # never refreshes
    monkeypatch.setitem(sys.modules, "amdsmi", fake)
    r = bench.sclk_during(_Torch(), lambda: time.sleep(0.002), seconds=0.1)
    assert r["mhz_median"] is None and "no fresh" in r["reason"]


def test_sclk_none_without_amdsmi(monkeypatch):
    monkeypatch.setitem(sys.modules, "amdsmi", None)                   # import raises ImportError
    r = bench.sclk_during(_Torch(), lambda: None, seconds=0.01)
    assert r["mhz_median"] is None and "amdsmi" in r["reason"]


def test_sclk_none_without_the_device(monkeypatch):
    fake, _ = _fake_amdsmi([_refresh(1, 100, [2000] * 8)])
    fake.amdsmi_get_gpu_device_bdf = lambda h: "0000:05:00.0"
    monkeypatch.setitem(sys.modules, "amdsmi", fake)
    r = bench.sclk_during(_Torch(), lambda: None, seconds=0.01)
    assert r["mhz_median"] is None and "0000:8b:00" in r["reason"]
