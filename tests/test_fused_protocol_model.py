"""CPU model of the fused decode kernel's work protocol (tests/fused_protocol_model.cpp).

Threads stand in for workgroups and their waves; the model replays the ticket
counter, the arrival counters, the bounded ready-word wait and the item slot
shared by a workgroup's waves, under random timing, and reports hangs (missed
barrier deadlines), workgroups split across two items, attention that read an
earlier call's selection, and inconsistent control words.

* The shipped protocol (ticket prefetch, two barriers around the item slot,
  epoch-valued ready words) and the variant without prefetch never hang, never
  split a workgroup and never read a stale selection, also when waits are
  abandoned (then the unit reports NaN and the next call is exact).
* Two hazards are shown, so that the checks are known to catch them: one barrier
  around the item slot (a skipped item's early `continue` lets thread 0 overwrite
  the slot before the other waves read it: workgroups split and barriers stop
  matching, the stall class of a persistent loop), and 0/1 ready flags reset by
  the last split (a flag raised late after an abandoned wait lets the next call
  attend over the previous call's selection).
"""
import os
import re
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("fpm") / "fused_protocol_model")
    subprocess.run(["g++", "-std=c++17", "-O1", "-pthread", os.path.join(HERE, "fused_protocol_model.cpp"), "-o", exe],
                   check=True)
    return exe


def run(exe, variant, trials, seed, spin):
    r = subprocess.run([exe, variant, str(trials), str(seed), str(spin)], capture_output=True, text=True,
                       timeout=240, check=True)
    return {k: int(v) for k, v in re.findall(r"(\w+)=(\d+)", r.stdout)}


@pytest.mark.parametrize("variant", ["shipped", "noprefetch"])
def test_protocol_sound_under_random_timing(model, variant):
    res = run(model, variant, 200, 11, 2)
    assert res["hang"] == 0 and res["mismatch"] == 0, res
    assert res["stale"] == 0 and res["wrong"] == 0, res
    assert res["timeouts"] > 0, f"the time-out path was not exercised: {res}"


def test_protocol_without_timeouts_is_exact(model):
    res = run(model, "shipped", 100, 12, 1 << 30)
    assert res == {**res, "hang": 0, "mismatch": 0, "stale": 0, "wrong": 0, "nan_units": 0, "timeouts": 0}, res


def test_one_barrier_item_slot_is_caught(model):
    res = run(model, "onebarrier", 15, 13, 1 << 30)
    assert res["hang"] + res["mismatch"] > 0, res


def test_zero_one_flags_let_a_late_flag_through(model):
    found = 0
    for seed in (2, 3, 4):
        found += run(model, "flags01", 300, seed, 2)["stale"]
        if found:
            break
    assert found > 0, "the stale-flag hazard of 0/1 ready flags was not reproduced"
