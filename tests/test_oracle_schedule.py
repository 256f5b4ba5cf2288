"""Pins for oracle.schedule: brute force, a hand-worked example, invariants."""
import math

import numpy as np
import pytest

from oracle.schedule import build_schedule, capacity, rows_cap
from tests.conftest import golden_path
from workloads import CONFIGS, make_inputs


def brute_force(top, E, mult, P, mb):
    """Dict-of-lists with Python's stable sorted(): an independent
    formulation of the schedule on tiny inputs."""
    T, k = len(top), len(top[0])
    C = min(T, math.ceil(float(np.float32(mult)) * T))
    per_expert = {e: [] for e in range(E)}
    invalid = 0
    for t in range(T):
        for j in range(k):
            e = int(top[t][j])
            if 0 <= e < E:
                per_expert[e].append(t * k + j)
            else:
                invalid += 1
    for e in per_expert:
        per_expert[e] = sorted(per_expert[e])
    offsets = [0]
    row_src = []
    slot_row = [-1] * (T * k)
    dropped = 0
    for e in range(E):
        keep = per_expert[e][:C]
        dropped += len(per_expert[e]) - len(keep)
        padded = -(-len(keep) // P) * P
        for q, a in enumerate(keep):
            slot_row[a] = offsets[-1] + q
        row_src += keep + [-1] * (padded - len(keep))
        offsets.append(offsets[-1] + padded)
    Rc = min(T * k, E * C) + E * (P - 1)
    row_src += [-1] * (Rc - len(row_src))
    mbs = T if mb <= 0 else mb
    n_mb = -(-T // mbs)
    mb_off = []
    for b in range(n_mb + 1):
        bound = min(b * mbs, T)
        row = []
        for e in range(E):
            keep = per_expert[e][:C]
            row.append(offsets[e] + sum(1 for a in keep if a // k < bound))
        mb_off.append(row)
    return dict(C=C, offsets=offsets, row_src=row_src, slot_row=slot_row, dropped=dropped,
                invalid=invalid, counts=[len(per_expert[e]) for e in range(E)], mb_offsets=mb_off,
                rows_cap=Rc)


def _check_equal(s, b):
    assert s["C"] == b["C"]
    assert s["rows_cap"] == b["rows_cap"]
    assert s["offsets"].tolist() == b["offsets"]
    assert s["row_src"].tolist() == b["row_src"]
    assert s["slot_row"].tolist() == b["slot_row"]
    assert s["dropped"] == b["dropped"] and s["invalid"] == b["invalid"]
    assert s["counts"].tolist() == b["counts"]
    assert s["mb_offsets"].tolist() == b["mb_offsets"]


@pytest.mark.parametrize("seed", range(40))
def test_schedule_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 40))
    k = int(rng.integers(1, 5))
    E = int(rng.integers(1, 9))
    P = int(rng.choice([1, 2, 4, 8, 32]))
    mult = float(rng.choice([0.1, 0.25, 0.5, 0.75, 1.0, 0.3]))
    mb = int(rng.choice([0, 1, 3, 7, 64]))
    # ids in [-1, E] so invalid ids and duplicates within a token occur
    top = rng.integers(-1, E + 1, size=(T, k)).astype(np.int64)
    s = build_schedule(top, E, mult, P, mb)
    _check_equal(s, brute_force(top.tolist(), E, mult, P, mb))


def _read_golden(name):
    d = {}
    for line in open(golden_path(name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        d[key] = vals
    return d


def test_schedule_hand_worked_example():
    g = _read_golden("schedule_small.txt")
    T, k, E, P, mb = (int(g[n][0]) for n in ("T", "k", "E", "P", "minibatch"))
    top = np.array([int(v) for v in g["top_experts"]], dtype=np.int64).reshape(T, k)
    s = build_schedule(top, E, float(g["mult"][0]), P, mb)
    ints = lambda n: [int(v) for v in g[n]]
    assert s["C"] == int(g["C"][0])
    assert s["rows_cap"] == int(g["rows_cap"][0])
    assert s["counts"].tolist() == ints("counts")
    assert s["kept"].tolist() == ints("kept")
    assert s["offsets"].tolist() == ints("offsets")
    assert s["row_src"].tolist() == ints("row_src")
    assert s["slot_row"].tolist() == ints("slot_row")
    assert s["dropped"] == int(g["dropped"][0]) and s["invalid"] == int(g["invalid"][0])
    assert s["n_mb"] == int(g["n_mb"][0])
    assert s["mb_offsets"].reshape(-1).tolist() == ints("mb_offsets")


def _invariants(s, top, E, mult):
    T, k = top.shape
    C = capacity(T, mult)
    valid = (top >= 0) & (top < E)
    assert s["counts"].sum() == T * k - s["invalid"] == valid.sum()
    assert s["kept"].sum() + s["dropped"] == s["counts"].sum()
    padded = s["offsets"][1:] - s["offsets"][:-1]
    assert np.all(padded % s["P"] == 0) and np.all(padded >= s["kept"]) and np.all(padded - s["kept"] < s["P"])
    assert s["offsets"][-1] <= s["rows_cap"] == rows_cap(T, k, E, mult, s["P"])
    # row_src / slot_row are mutually inverse on kept assignments
    kept_a = np.nonzero(s["slot_row"] >= 0)[0]
    assert np.all(s["row_src"][s["slot_row"][kept_a]] == kept_a)
    rs = s["row_src"]
    assert np.all(s["slot_row"][rs[rs >= 0]] == np.nonzero(rs >= 0)[0])
    # segments ascending in flat order, right expert, first C of that expert
    for e in range(E):
        seg = rs[s["offsets"][e]: s["offsets"][e] + s["kept"][e]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(top.reshape(-1)[seg] == e)
        assert np.all(rs[s["offsets"][e] + s["kept"][e]: s["offsets"][e + 1]] == -1)
        assert s["kept"][e] == min(C, s["counts"][e])
    if mult >= 1.0:
        assert s["dropped"] == 0


@pytest.mark.parametrize("name", list(CONFIGS))
def test_schedule_invariants_on_configs(name):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg.with_(H=32, I=32, I_s=32 if cfg.I_s else 0), with_grad=False)
    mults = [cfg.capacity_multiplier] + ([0.5] if cfg.routing == "zipf" else [])
    for mult in mults:
        s = build_schedule(inp["top_experts"], cfg.E, mult, cfg.expert_pad)
        _invariants(s, inp["top_experts"], cfg.E, mult)
        # "the schedule table is at most a few megabytes" ([R] §Tuning...):
        nbytes = 4 * (s["row_src"].size + s["slot_row"].size + 3 * cfg.E)
        assert nbytes < 8 << 20


def test_skewed_config_drops_at_half_capacity():
    """The Zipf-skewed workload overflows its hottest experts at mult 0.5
    and drops nothing at 1.0."""
    cfg = CONFIGS["skew_bf16_fwd"]
    inp = make_inputs(cfg.with_(H=32, I=32, I_s=32), with_grad=False)
    s1 = build_schedule(inp["top_experts"], cfg.E, 1.0, 32)
    s5 = build_schedule(inp["top_experts"], cfg.E, 0.5, 32)
    assert s1["dropped"] == 0
    frac = s5["dropped"] / (cfg.T * cfg.k)
    assert 0.10 < frac < 0.25
    assert s5["counts"][0] == s5["counts"].max()


def test_minibatch_size_does_not_change_permutation():
    rng = np.random.default_rng(7)
    top = rng.integers(0, 6, size=(100, 3)).astype(np.int64)
    base = build_schedule(top, 6, 0.4, 8, 0)
    for mb in (1, 7, 33, 100, 1000):
        s = build_schedule(top, 6, 0.4, 8, mb)
        assert np.array_equal(s["row_src"], base["row_src"])
        assert np.array_equal(s["slot_row"], base["slot_row"])
        assert np.array_equal(s["mb_offsets"][0], s["offsets"][:-1])
        assert np.array_equal(s["mb_offsets"][-1], s["offsets"][:-1] + s["kept"])


def test_capacity_float32_reading():
    # the multiplier is a float32 config field; 0.4f * 5 = 2.0000000298 -> 3
    assert capacity(5, 0.4) == 3
    assert capacity(16384, 0.5) == 8192
    assert capacity(100, 1.0) == 100
    assert capacity(100, 2.0) == 100
