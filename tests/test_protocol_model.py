"""CPU model of the persistent kernels' work-distribution protocol.

tests/protocol_model/protocol_model.cpp runs the kernels' protocol -- atomic
role tickets, queue counters, epoch-valued flags published by arrival
counters with release order and awaited with acquire order, bounded waits
that record a timeout and abort the launch, and the last workgroup's reset
of the launch counters -- with one std::thread per workgroup and a limit on
how many run at once (the GPU's residency).  These tests check, on the CPU:

* every operation finishes with the right data when every workgroup is
  resident, for any role split, landing order and number of launches in a
  row on the same control memory (stale flags of an earlier launch never
  satisfy a later one, and the counters are back at zero after each launch);
* workgroups that start late, with fewer slots than workgroups, still finish
  (land and reduce tickets come first and never wait on compute);
* a unit that never lands makes the waiters time out and every workgroup
  exit, instead of hanging;
* the MoE combine's wait for the last tile needs no co-residency while land
  workgroups take tiles too (the library's default), and hangs without it
  when they keep their role (static roles), which is why the library caps
  that launch's grid at the residency.
"""
import json
import os
import shutil
import subprocess

import pytest

SRC = os.path.join(os.path.dirname(__file__), "protocol_model", "protocol_model.cpp")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path_factory.mktemp("protocol_model") / "protocol_model")
    subprocess.run([gxx, "-O2", "-std=c++17", "-pthread", "-Wall", "-Werror", SRC, "-o", exe], check=True)

    def run(op, *args):
        out = subprocess.run([exe, op, *map(str, args)], capture_output=True, text=True, timeout=120)
        assert out.returncode == 0, out.stderr
        return json.loads(out.stdout.strip().splitlines()[-1])

    return run


@pytest.mark.parametrize("land", [1, 2, 8])
@pytest.mark.parametrize("help_", [True, False])
def test_ag_role_splits_and_landing_order(model, land, help_):
    args = ["--land", land, "--permute", "--launches", 4]
    if not help_:
        args.append("--no-help")
    r = model("ag", *args)
    assert r["ok"], r


def test_ag_late_starters_with_fewer_slots(model):
    r = model("ag", "--grid", 48, "--slots", 4, "--land", 2, "--late-us", 2000, "--permute", "--no-help")
    assert r["ok"], r
    # helpers land too, so no land role is needed when compute helps
    r = model("ag", "--grid", 48, "--slots", 4, "--land", 0, "--late-us", 2000)
    assert r["ok"], r


def test_ag_without_land_role_or_helpers_hangs(model):
    # nobody lands: the compute workgroups' waits must end in a timeout
    r = model("ag", "--grid", 16, "--slots", 4, "--land", 0, "--no-help", "--timeout-ms", 200, "--launches", 1)
    assert not r["ok"] and r["err"] == 2, r


@pytest.mark.parametrize("op,extra", [("ag", []), ("rs", ["--land", 4]), ("moe", []), ("ring", ["--land", 4])])
def test_withheld_unit_times_out(model, op, extra):
    r = model(op, "--withhold", 3, "--timeout-ms", 150, "--launches", 1, *extra)
    assert not r["ok"] and r["err"] == 2 and r["mismatch"] == 0, r


def test_epochs_across_many_launches(model):
    for op, extra in [("ag", []), ("rs", ["--land", 4]), ("moe", ["--combine"]), ("ring", ["--land", 4])]:
        r = model(op, "--launches", 25, "--permute", "--late-us", 300, *extra)
        assert r["ok"], (op, r)


@pytest.mark.parametrize("compute", [-1, 0])
def test_rs_reduce_role_and_transfer_alone(model, compute):
    r = model("rs", "--land", 6, "--items", 24, "--tiles", 72, "--compute", compute, "--grid", 32, "--slots", 8,
              "--late-us", 1000)
    assert r["ok"], r


def test_moe_route_scan_land_compute(model):
    r = model("moe", "--grid", 40, "--slots", 40, "--items", 64, "--tiles", 96, "--late-us", 1000)
    assert r["ok"], r
    r = model("moe", "--grid", 40, "--slots", 6, "--land", 2, "--items", 64, "--tiles", 96, "--late-us", 1000)
    assert r["ok"], r


def test_moe_combine_residency(model):
    # all resident: fine either way
    for extra in ([], ["--static"]):
        r = model("moe", "--combine", "--grid", 24, "--slots", 24, "--land", 4, "--late-us", 1000, *extra)
        assert r["ok"], r
    # land workgroups that take tiles too: a workgroup in the combine has seen
    # the tile queue empty, so any number of slots suffices
    r = model("moe", "--combine", "--grid", 24, "--slots", 4, "--land", 4, "--late-us", 1000)
    assert r["ok"], r
    # static roles: the land workgroups fill every slot and wait for tiles
    # nobody runs (why the library keeps that launch within one residency)
    r = model("moe", "--combine", "--static", "--grid", 24, "--slots", 4, "--land", 4, "--timeout-ms", 200,
              "--launches", 1)
    assert not r["ok"] and r["err"] == 2, r


def test_ring_pair_merge(model):
    r = model("ring", "--grid", 24, "--slots", 6, "--land", 4, "--tiles", 64, "--items", 40, "--late-us", 2000,
              "--permute")
    assert r["ok"], r
