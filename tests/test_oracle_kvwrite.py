"""Pins for the oracle's KV-pool writer (CPU only).

The int8 tensor-core prefill attention page, section "Why the attention, and
why tensor cores", gives the pool this path reads: 16-token int8 pages, rows
token-major, one scale per token and KV head.  The writer quantizes each
(token, head) row with the page's per-row formula and stores it at the
token's slot.  The pins: a hand-worked fixture (tests/golden), rows already on
the int8 grid (codes equal the inputs, so the layout is checked without the
formula), the per-element round-trip bound, and skipped or untouched slots.
"""
import json
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_write_example.json")


def _empty_pool(pages, hkv, fill=0):
    kp = np.full((pages, 16, hkv, 256), fill, dtype=np.int8)
    sc = np.full((pages, 16, hkv), np.float32(-1.0), dtype=np.float32)
    return kp, kp.copy(), sc, sc.copy()


def test_hand_worked_fixture():
    g = json.load(open(GOLDEN))
    k = np.zeros((2, 2, 256), dtype=np.float32)
    v = np.zeros((2, 2, 256), dtype=np.float32)
    for r in g["k_rows"]:
        k[r["token"], r["head"], r["channels"]] = r["values"]
    for r in g["v_rows"]:
        v[r["token"], r["head"], r["channels"]] = r["values"]
    kp, vp, ks, vs = oracle.kv_write_i8(k, v, np.array(g["slots"]), *_empty_pool(2, 2, fill=99))
    for e in g["expect"]:
        pool, sc = (kp, ks) if e["pool"] == "k" else (vp, vs)
        row = pool[e["page"], e["pos"], e["head"]]
        if "codes_0_4" in e:
            assert row[:4].tolist() == e["codes_0_4"]
            assert np.all(row[4:] == 0)
        else:
            assert row[5:7].tolist() == e["codes_5_7"]
            assert np.all(np.delete(row, [5, 6]) == 0)
        assert sc[e["page"], e["pos"], e["head"]] == np.float32(e["scale_num"]) / np.float32(e["scale_den"])
    # the written slots' other head rows are zero rows; every other slot is untouched
    written = {(1, 1), (0, 3)}
    for page in range(2):
        for pos in range(16):
            if (page, pos) not in written:
                assert np.all(kp[page, pos] == 99) and np.all(vp[page, pos] == 99)
                assert np.all(ks[page, pos] == -1.0) and np.all(vs[page, pos] == -1.0)


def test_rows_on_the_int8_grid_land_at_their_slots():
    # integer rows holding a +-127: codes are the integers and the scale is 1,
    # so the pool must hold exactly the input at [slot // 16][slot % 16][head]
    rng = np.random.default_rng(11)
    n, hkv, pages = 40, 3, 5
    k = rng.integers(-126, 127, size=(n, hkv, 256)).astype(np.float32)
    v = rng.integers(-126, 127, size=(n, hkv, 256)).astype(np.float32)
    k[:, :, 7] = 127.0
    v[:, :, 200] = -127.0
    slots = rng.permutation(pages * 16)[:n]
    kp, vp, ks, vs = oracle.kv_write_i8(k, v, slots, *_empty_pool(pages, hkv))
    for t, s in enumerate(slots):
        for h in range(hkv):
            assert np.array_equal(kp[s // 16, s % 16, h].astype(np.float32), k[t, h])
            assert np.array_equal(vp[s // 16, s % 16, h].astype(np.float32), v[t, h])
            assert ks[s // 16, s % 16, h] == 1.0 and vs[s // 16, s % 16, h] == 1.0


def test_round_trip_bound_and_full_scale():
    kb, vb, k, v, slots, kp0, vp0, ks0, vs0 = workloads.make_kv_rows(50, 2, 4, seed=5)
    kp, vp, ks, vs = oracle.kv_write_i8(k, v, slots, kp0, vp0, ks0, vs0)
    for x, pool, sc in ((k, kp, ks), (v, vp, vs)):
        got = pool[slots // 16, slots % 16].astype(np.float64)  # [n][hkv][256]
        step = sc[slots // 16, slots % 16].astype(np.float64)[..., None]
        # half a step, plus float32 rounding of 127/amax and of x * (127/amax)
        # (each below 2^-23 relative, on values up to 127 steps)
        assert np.all(np.abs(got * step - x) <= step * (0.5 + 127 * 2.0**-21))
        assert np.all(np.abs(got).max(axis=-1) == 127)


def test_out_of_range_slots_are_skipped():
    kb, vb, k, v, slots, kp0, vp0, ks0, vs0 = workloads.make_kv_rows(6, 1, 1, seed=9)
    slots = slots.copy()
    slots[1], slots[4] = -1, 16  # outside [0, 16 * 1)
    kp, vp, ks, vs = oracle.kv_write_i8(k, v, slots, kp0, vp0, ks0, vs0)
    touched = set(slots[[0, 2, 3, 5]].tolist())
    for pos in range(16):
        same = np.array_equal(kp[0, pos], kp0[0, pos]) and ks[0, pos, 0] == ks0[0, pos, 0]
        assert same == (pos not in touched)
