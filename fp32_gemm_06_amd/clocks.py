"""Graphics-clock samples taken while the benchmark's timed loops run.

The FP32 matrix peak (256 CUs x 256 FLOP/clk x 2.4 GHz) assumes the top
graphics clock; a long MFMA loop can run below it.  This module reads the
current graphics clock of the benchmarked GPU from the kernel driver's sysfs
table (``pp_dpm_sclk``: one line per level, the current one marked ``*``) in
a background thread and groups the samples by the phase the benchmark is in.
It only reads files; when the table is absent or unreadable it reports why
and the benchmark carries on without clock data.
"""
from __future__ import annotations

import glob
import os
import re
import statistics
import threading
import time


def _card_for(pci_domain: int, pci_bus: int, pci_device: int):
    """The sysfs device directory of the GPU at this PCI address, or None."""
    want = f"{pci_domain:04x}:{pci_bus:02x}:{pci_device:02x}."
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            slot = os.path.basename(os.path.realpath(dev))
        except OSError:
            continue
        if slot.lower().startswith(want):
            return dev
    return None


def _current_mhz(path: str):
    with open(path) as f:
        for line in f:
            if "*" in line:
                m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                if m:
                    return int(m.group(1))
    return None


class ClockSampler:
    """Samples the graphics clock every ``period`` seconds in a daemon thread.

    ``phase(name)`` tags the following samples; ``summary()`` gives, per
    phase, the number of samples and the median / min / max clock in MHz.
    """

    def __init__(self, pci_domain: int, pci_bus: int, pci_device: int, period: float = 0.002):
        self.period = period
        self.samples: dict[str, list[int]] = {}
        self.error = None
        self._phase = None
        self._stop = threading.Event()
        self._thread = None
        dev = _card_for(pci_domain, pci_bus, pci_device)
        self.path = os.path.join(dev, "pp_dpm_sclk") if dev else None
        if self.path is None:
            self.error = "no sysfs device for the GPU's PCI address"
        else:
            try:
                if _current_mhz(self.path) is None:
                    self.error = f"{self.path} has no current level"
            except OSError as e:
                self.error = f"{self.path}: {e.strerror}"

    def start(self):
        if self.error is None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def _run(self):
        while not self._stop.is_set():
            ph = self._phase
            if ph is not None:
                try:
                    mhz = _current_mhz(self.path)
                except OSError:
                    mhz = None
                if mhz is not None:
                    self.samples.setdefault(ph, []).append(mhz)
            time.sleep(self.period)

    def phase(self, name):
        self._phase = name

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=1.0)

    def summary(self):
        if self.error is not None:
            return {"source": "pp_dpm_sclk", "error": self.error}
        out = {"source": self.path}
        for ph, v in self.samples.items():
            out[ph] = {"samples": len(v), "median_mhz": statistics.median(v), "min_mhz": min(v),
                       "max_mhz": max(v)}
        return out


def cpu_model() -> str:
    """The host CPU's model name (what ``lscpu`` prints), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"
