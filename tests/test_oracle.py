"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
printed figure, a hand-derived value, a library routine (numpy / torch number
conversions), an algebraic invariant of the trellis, or exhaustive search.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LUT = workload.lut_fp16(0)


def golden_rows(name: str) -> list[list[str]]:
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def lut_pair(idx: int, neg: int) -> tuple[int, int]:
    p0, p1 = int(LUT[idx, 0]), int(LUT[idx, 1])
    if neg:
        p0 ^= 0x8000
        p1 ^= 0x8000
    return p0, p1


# ---------------------------------------------------------------------------
# storage: b + 16/d bits per parameter (onedev.kr, "How it works")
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("kv", [3, 4, 5, 6])
def test_record_size_is_rate_plus_one_scale(d, kv):
    R = oracle.record_bytes(d, kv)
    b = kv / 2  # V = 2 outputs per kv-bit step
    assert R * 8 == b * d + 16
    assert R * 8 / d == pytest.approx(b + 16 / d, abs=0)


def test_record_sizes_of_the_workloads():
    assert [oracle.record_bytes(64, 4), oracle.record_bytes(256, 4), oracle.record_bytes(512, 4)] == [18, 66, 130]
    assert [oracle.record_bytes(512, kv) for kv in (3, 4, 5, 6)] == [98, 130, 162, 194]
    # whole-byte codes only for records
    assert oracle.record_bytes(10, 4) == 0 and oracle.code_bits(10, 4) == 20
    assert oracle.code_bits(6, 4) == 0  # fewer code bits than one window


def test_storage_figures_printed_on_the_pages():
    g = {k: float(v) for k, v in golden_rows("storage.txt")}
    ratio = g["original_gb"] / g["cp_gb"]
    # an FP8 table at b + 16/d bits per parameter shrinks by 8/(2 + 16/d) < 4,
    # approaching 4 for long rows: the printed 202.7 -> 50.7 GB is just under 4x
    for d in (64, 256, 512, 4096):
        r = g["original_bits_per_param"] / (oracle.record_bytes(d, 4) * 8 / d)
        assert 3.5 < r < 4.0
        # against 16-bit originals the same code gives just under 8x
        assert 7.0 < 2 * r < 8.0
    assert 3.9 < ratio <= 4.0
    assert g["compression_low"] <= ratio * (1 + 1e-3) and 2 * ratio <= g["compression_high"]
    # 50.7 GB over 4 GPUs is the 12.7 GB per GPU the pages print, and the one-GPU
    # workload's 97,690,000 records of 130 bytes reproduce it
    assert g["cp_gb"] / g["gpus"] == pytest.approx(g["per_gpu_gb_4gpu"], abs=0.05)
    cfg = workload.CONFIGS["gpu_d512"]
    assert cfg.rows * oracle.record_bytes(512, 4) / 1e9 == pytest.approx(g["per_gpu_gb_4gpu"], abs=0.01)


# ---------------------------------------------------------------------------
# number formats: against numpy / torch conversions
# ---------------------------------------------------------------------------

def test_fp16_values_match_numpy_exhaustively():
    vals = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_double(h) for h in range(65536)])
    same = (got == vals) | (np.isnan(got) & np.isnan(vals))
    assert same.all()
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_bf16_values_match_torch_exhaustively():
    ref = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_double(b) for b in range(65536)])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    # every finite pattern survives value -> bf16
    back = np.array([oracle.bf16_from_double(v) for v in got])
    finite = ~np.isnan(got)
    assert (back[finite] == np.arange(65536)[finite]).all()


def test_bf16_rounding_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    # force exact ties on a third of them, and subnormals on some
    bits[::3] = (bits[::3] & 0xFFFF0000) | 0x8000
    bits[1::7] &= 0x807FFFFF
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_double(float(v)) for v in x], dtype=np.uint16)
    assert (got == ref).all()


def test_bf16_rounding_is_single_from_the_exact_value():
    # 1 + 2^-8 + 2^-30 lies above the midpoint of 1 and 1 + 2^-7; a detour
    # through float32 would make it a tie and round down to 1.0
    assert oracle.bf16_from_double(1 + 2**-8 + 2**-30) == 0x3F81
    assert oracle.bf16_from_double(1 + 2**-8) == 0x3F80          # tie -> even
    assert oracle.bf16_from_double(1 + 3 * 2**-8) == 0x3F82      # tie -> even (up)
    assert oracle.bf16_from_double(-0.0) == 0x8000
    assert oracle.bf16_from_double(2.0**-133) == 0x0001          # smallest subnormal
    assert oracle.bf16_from_double(2.0**-134) == 0x0000          # tie -> even (zero)
    assert oracle.bf16_from_double(3 * 2.0**-134) == 0x0002      # tie -> even (up)
    assert oracle.bf16_from_double(3.4e38) == 0x7F80             # rounds past the largest finite
    assert oracle.bf16_from_double(float.fromhex("0x1.fep127")) == 0x7F7F


# ---------------------------------------------------------------------------
# the trellis rule: hand-derived windows and closed forms
# ---------------------------------------------------------------------------

def test_worked_windows():
    for d, kv, code_hex, t, s_hex, idx, neg in golden_rows("worked_windows.txt"):
        d, kv, t, idx, neg = int(d), int(kv), int(t), int(idx), int(neg)
        code = np.frombuffer(bytes.fromhex(code_hex), dtype=np.uint8)
        s = oracle.window(code, d, kv, t)
        assert s == int(s_hex, 16), (code_hex, t)
        assert oracle.hash_window(s) == (idx, neg)
        f = oracle.decode_code(LUT, code, d, kv)
        assert (int(f[2 * t]), int(f[2 * t + 1])) == lut_pair(idx, neg)


@pytest.mark.parametrize("d", [64, 512])
def test_constant_nibble_codes_give_one_pair(d):
    for p, idx, neg in golden_rows("constant_codes_kv4.txt"):
        p, idx, neg = int(p), int(idx), int(neg)
        code = np.full(d // 4, p | (p << 4), dtype=np.uint8)
        f = oracle.decode_code(LUT, code, d, 4)
        p0, p1 = lut_pair(idx, neg)
        assert (f[0::2] == p0).all() and (f[1::2] == p1).all(), p


def test_hash_invariants_exhaustive():
    idx = np.empty(65536, dtype=np.int64)
    neg = np.empty(65536, dtype=np.int64)
    for s in range(65536):
        idx[s], neg[s] = oracle.hash_window(s)
    # every output index is reached by 128 windows, every signed output by 64
    assert (np.bincount(idx, minlength=512) == 128).all()
    assert (np.bincount(idx * 2 + neg, minlength=1024) == 64).all()
    s = np.arange(65536)
    # flipping the top bit flips the sign and bit 8 of the index
    assert (idx[s ^ 0x8000] == idx ^ 256).all() and (neg[s ^ 0x8000] == 1 - neg).all()
    # the complement window selects the same entry with the other sign
    assert (idx[s ^ 0xFFFF] == idx).all() and (neg[s ^ 0xFFFF] == 1 - neg).all()
    # negation is bit 15 of the window
    assert (neg == (s >> 15)).all()


def _code_int(code: np.ndarray) -> int:
    return int.from_bytes(code.tobytes(), "little")


def _int_code(v: int, nbytes: int) -> np.ndarray:
    return np.frombuffer(v.to_bytes(nbytes, "little"), dtype=np.uint8).copy()


shapes = st.sampled_from([(16, 4), (32, 3), (64, 4), (64, 3), (64, 5), (64, 6), (128, 5),
                          (256, 4), (512, 3), (512, 6)])


@settings(max_examples=60, deadline=None)
@given(shape=shapes, seed=st.integers(0, 2**32 - 1))
def test_complement_code_negates_the_row(shape, seed):
    d, kv = shape
    nb = oracle.code_bits(d, kv) // 8
    code = np.random.default_rng(seed).integers(0, 256, nb, dtype=np.uint8)
    f = oracle.decode_code(LUT, code, d, kv)
    g = oracle.decode_code(LUT, code ^ 0xFF, d, kv)
    assert (g == (f ^ 0x8000)).all()


@settings(max_examples=60, deadline=None)
@given(shape=shapes, seed=st.integers(0, 2**32 - 1), r=st.integers(0, 300))
def test_rotating_the_code_rotates_the_row(shape, seed, r):
    # tail-biting: the trellis has no start; rotating the code by whole steps
    # rotates the output by the same number of steps
    d, kv = shape
    N = oracle.code_bits(d, kv)
    T = d // 2
    r %= T
    code = np.random.default_rng(seed).integers(0, 256, N // 8, dtype=np.uint8)
    v = _code_int(code)
    sh = kv * r
    rot = ((v >> sh) | (v << (N - sh))) & ((1 << N) - 1)
    f = oracle.decode_code(LUT, code, d, kv)
    g = oracle.decode_code(LUT, _int_code(rot, N // 8), d, kv)
    assert (g == np.roll(f, -2 * r)).all()


def test_single_bit_touches_only_its_windows():
    # a bitshift trellis: code bit j enters exactly the 16 / kv windows that
    # cover it, i.e. steps whose window [kv(t+1)-16, kv(t+1)) contains j
    for d, kv in [(64, 4), (64, 3), (512, 6)]:
        N = oracle.code_bits(d, kv)
        base = np.zeros(N // 8, dtype=np.uint8)
        f0 = oracle.decode_code(LUT, base, d, kv)
        for j in (0, 1, N // 2 + 3, N - 1):
            c = base.copy()
            c[j >> 3] |= 1 << (j & 7)
            f1 = oracle.decode_code(LUT, c, d, kv)
            changed = set(np.nonzero((f1 != f0).reshape(-1, 2).any(axis=1))[0].tolist())
            covering = {t for t in range(d // 2)
                        if any(((kv * (t + 1) - 16 + m) % N) == j for m in range(16))}
            assert changed <= covering
            assert len(covering) in (16 // kv, 16 // kv + 1)


# ---------------------------------------------------------------------------
# scaled rows: exact product, one round-to-nearest-even (against torch)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,kv", [(64, 4), (256, 4), (512, 3), (512, 6)])
def test_scaled_rows_match_torch_fp32_product(d, kv):
    recs = workload.random_records(64, d, kv, seed=11)
    nb = oracle.code_bits(d, kv) // 8
    # include a few special scales: 1, a power of two, negative, zero
    specials = [0x3F80, 0x4100, 0xBF00, 0x0000, 0x8000]
    for i, a in enumerate(specials):
        recs[i, nb] = a & 0xFF
        recs[i, nb + 1] = a >> 8
    for rec in recs:
        y = oracle.decode_record(LUT, rec, d, kv)
        f = torch.from_numpy(oracle.decode_code(LUT, rec[:nb], d, kv).astype(np.int16)).view(torch.float16)
        a = int(rec[nb]) | (int(rec[nb + 1]) << 8)
        alpha = torch.tensor([a], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
        ref = (f.float() * alpha).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert (y == ref).all()


# ---------------------------------------------------------------------------
# the lookup: requested rows, in the original order
# ---------------------------------------------------------------------------

def test_lookup_returns_requested_rows_in_order():
    d, kv, rows = 64, 4, 300
    recs = workload.random_records(rows, d, kv, seed=12)
    ids = np.array([5, 299, 0, 5, 5, 17, -1, 300, 1 << 40, 123, 0], dtype=np.int64)
    for raw in (False, True):
        out, bad = oracle.lookup_decode(LUT, recs, rows, d, kv, ids, raw=raw, nthreads=3)
        assert bad == 3
        for j, i in enumerate(ids):
            if 0 <= i < rows:
                exp = (oracle.decode_code(LUT, recs[i, : kv * d // 16], d, kv) if raw
                       else oracle.decode_record(LUT, recs[i], d, kv))
                assert (out[j] == exp).all()
            else:
                assert (out[j] == 0).all()
    out, bad = oracle.lookup_decode(LUT, recs, rows, d, kv, np.zeros(0, np.int64))
    assert out.shape == (0, d) and bad == 0


def test_lookup_reads_only_its_own_record():
    # records are independently addressable: garbage in the neighbours of a
    # record does not change its row
    d, kv, rows = 256, 4, 9
    recs = workload.random_records(rows, d, kv, seed=13)
    ids = np.array([4], dtype=np.int64)
    a, _ = oracle.lookup_decode(LUT, recs, rows, d, kv, ids)
    recs2 = recs.copy()
    recs2[3] ^= 0xA5
    recs2[5] ^= 0x5A
    b, _ = oracle.lookup_decode(LUT, recs2, rows, d, kv, ids)
    assert (a == b).all()


# ---------------------------------------------------------------------------
# encoder: brute force, planted codewords, tail-biting, the norm rule
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,kv", [(8, 4), (10, 4), (12, 4), (12, 3), (16, 3), (8, 5), (8, 6)])
def test_exact_tcq_equals_exhaustive_search(d, kv):
    rng = np.random.default_rng(1000 + 10 * d + kv)
    for _ in range(2):
        z = rng.standard_normal(d)
        best, _ = oracle.bruteforce_min(z, d, kv, LUT)
        enc = oracle.tcq_encode(z, d, kv, LUT, oracle.ENC_EXACT)
        assert enc.certified
        assert enc.cost == pytest.approx(best, rel=1e-12, abs=1e-15)
        # the path metric is the distortion of the code as the decoder reads it
        assert oracle.distortion(z, LUT, enc.code, d, kv) == pytest.approx(enc.cost, rel=1e-12)
        heur = oracle.tcq_encode(z, d, kv, LUT, oracle.ENC_HEURISTIC)
        assert heur.cost >= best * (1 - 1e-12)
        assert oracle.distortion(z, LUT, heur.code, d, kv) == pytest.approx(heur.cost, rel=1e-12)


@pytest.mark.parametrize("d,kv,mode", [(64, 4, oracle.ENC_EXACT), (64, 3, oracle.ENC_EXACT),
                                       (256, 4, oracle.ENC_HEURISTIC),
                                       (512, 6, oracle.ENC_HEURISTIC)])
def test_planted_codeword_is_recovered(d, kv, mode):
    rng = np.random.default_rng(d + kv)
    N = oracle.code_bits(d, kv)
    code = rng.integers(0, 256, N // 8, dtype=np.uint8)
    z = np.array([oracle.fp16_to_double(h) for h in oracle.decode_code(LUT, code, d, kv)])
    enc = oracle.tcq_encode(z, d, kv, LUT, mode)
    assert enc.cost == 0.0
    z2 = np.array([oracle.fp16_to_double(h) for h in oracle.decode_code(LUT, enc.code, d, kv)])
    assert (z2 == z).all()


@pytest.mark.parametrize("d,kv", [(64, 4), (256, 4), (64, 6)])
def test_heuristic_codes_are_consistent_tail_biting_paths(d, kv):
    rng = np.random.default_rng(3)
    for _ in range(3):
        z = rng.standard_normal(d)
        enc = oracle.tcq_encode(z, d, kv, LUT, oracle.ENC_HEURISTIC)
        assert oracle.distortion(z, LUT, enc.code, d, kv) == pytest.approx(enc.cost, rel=1e-12)
        ex = oracle.tcq_encode(z, d, kv, LUT, oracle.ENC_EXACT, max_starts=4)
        assert ex.cost <= enc.cost
        assert oracle.distortion(z, LUT, ex.code, d, kv) == pytest.approx(ex.cost, rel=1e-12)


@pytest.mark.parametrize("d,kv", [(12, 4), (16, 3), (8, 5), (8, 6)])
def test_heuristic_code_is_best_among_codes_with_its_start_memory(d, kv):
    # The heuristic's second pass is a Viterbi search from one start memory W
    # that keeps the paths ending in W (onedev.kr, "How it works": the code is
    # a tail-biting path). Its result must therefore be the exhaustive minimum
    # of ||z - f(c)||^2 over every code whose memory before step 0 is W. That
    # memory is the 16 - kv oldest bits of the window of step 0, which are
    # the last 16 - kv bits of the circular code.
    N = oracle.code_bits(d, kv)
    M = 16 - kv
    rng = np.random.default_rng(4000 + 10 * d + kv)
    for _ in range(2):
        z = rng.standard_normal(d)
        heur = oracle.tcq_encode(z, d, kv, LUT, oracle.ENC_HEURISTIC)
        bits = np.unpackbits(heur.code, bitorder="little")[:N]
        best = np.inf
        for free in range(1 << (N - M)):
            b = bits.copy()
            b[:N - M] = (free >> np.arange(N - M)) & 1
            code = np.packbits(b, bitorder="little")
            best = min(best, oracle.distortion(z, LUT, code, d, kv))
        assert heur.cost == pytest.approx(best, rel=1e-12, abs=1e-15)
        # and the exhaustive minimum over all codes is no larger
        full, _ = oracle.bruteforce_min(z, d, kv, LUT)
        assert full <= best * (1 + 1e-12)


def test_heuristic_start_memory_is_that_of_the_best_rotated_free_start_path():
    # The heuristic's first pass searches, from every start memory, the
    # steps in the order T/2, ..., T-1, 0, ..., T/2-1, and takes the memory
    # its best path holds just before step 0. Brute force at d = 8, kv = 4:
    # a free-start path over the T = 4 rotated steps is any 28-bit string,
    # whose k-th window is bits [4k, 4k + 16); the memory before step 0
    # (visited as k = T - T/2) is bits [4(T - T/2), 4(T - T/2) + 12). It
    # must be the start memory of the heuristic's code, its last 12 bits.
    # Branch costs follow the trellis reading of the decoder: +-LUT[idx] with
    # idx and the sign from the window hash, fp16 values taken by numpy.
    d, kv = 8, 4
    T, M = d // 2, 16 - kv
    rot = T // 2
    N = oracle.code_bits(d, kv)
    idx = np.empty(65536, dtype=np.int64)
    neg = np.empty(65536, dtype=np.int64)
    for w in range(65536):
        idx[w], neg[w] = oracle.hash_window(w)
    g = LUT.view(np.float16).astype(np.float64)[idx]
    g[neg == 1] *= -1.0
    rng = np.random.default_rng(5)
    for _ in range(2):
        z = rng.standard_normal(d)
        step_cost = [(z[2 * t] - g[:, 0]) ** 2 + (z[2 * t + 1] - g[:, 1]) ** 2 for t in range(T)]
        order = [(k + rot) % T for k in range(T)]
        best, arg = np.inf, []
        chunk = 1 << 22
        for base in range(0, 1 << (M + T * kv), chunk):
            b = np.arange(base, base + chunk, dtype=np.int64)
            tot = step_cost[order[0]][b & 0xFFFF]
            for k in range(1, T):
                tot = tot + step_cost[order[k]][(b >> (kv * k)) & 0xFFFF]
            m = tot.min()
            if m < best:
                best, arg = m, list(base + np.nonzero(tot == m)[0])
            elif m == best:
                arg += list(base + np.nonzero(tot == m)[0])
        assert len(arg) == 1  # a unique best path for these seeds: no tie rule involved
        w_best = (int(arg[0]) >> (kv * (T - rot))) & ((1 << M) - 1)
        heur = oracle.tcq_encode(z, d, kv, LUT, oracle.ENC_HEURISTIC)
        w_code = (_code_int(heur.code) >> (N - M)) & ((1 << M) - 1)
        assert w_code == w_best


def test_norm_restoring_scale():
    # alpha = ||e|| / ||f(c)|| (onedev.kr, "How it differs"): with the exact
    # alpha the rebuilt row has the original norm; with the stored bf16 alpha
    # and bf16 outputs the norm is off by at most 2^-9 (alpha) + 2^-9 (outputs)
    d, kv = 256, 4
    e = workload.gaussian_rows(16, d, seed=21)
    recs, infos = oracle.encode_rows(e, d, kv, LUT, oracle.ENC_HEURISTIC)
    for i in range(e.shape[0]):
        rec, _, alpha = oracle.encode_row(e[i], d, kv, LUT, oracle.ENC_HEURISTIC)
        assert (rec == recs[i]).all()
        nb = oracle.code_bits(d, kv) // 8
        f = np.array([oracle.fp16_to_double(h) for h in oracle.decode_code(LUT, rec[:nb], d, kv)])
        ne = np.linalg.norm(e[i])
        assert np.linalg.norm(alpha * f) == pytest.approx(ne, rel=1e-12)
        a_bits = int(rec[nb]) | (int(rec[nb + 1]) << 8)
        assert a_bits == oracle.bf16_from_double(alpha)
        y = np.array([oracle.bf16_to_double(b) for b in oracle.decode_record(LUT, rec, d, kv)])
        assert abs(np.linalg.norm(y) / ne - 1) <= 2.0**-8


def test_zero_row_encodes_to_zero_scale():
    rec, info, alpha = oracle.encode_row(np.zeros(64), 64, 4, LUT)
    assert alpha == 0.0 and (rec == 0).all()


def test_distortion_between_rate_distortion_bound_and_scalar_quantiser():
    # sanity of the encoder at 2 bits per element on N(0,1) data: per-element
    # MSE of z above the Gaussian rate-distortion bound 2^-4 and below the
    # 2-bit Lloyd-Max scalar quantiser's 0.1175
    d, kv = 256, 4
    e = workload.gaussian_rows(24, d, seed=22)
    z = e / np.linalg.norm(e, axis=1, keepdims=True) * np.sqrt(d)
    costs = [oracle.tcq_encode(zi, d, kv, LUT, oracle.ENC_HEURISTIC).cost for zi in z]
    mse = float(np.mean(costs)) / d
    assert 0.0625 < mse < 0.1175, mse


# ---------------------------------------------------------------------------
# mixed-rate tables (reading R11)
# ---------------------------------------------------------------------------

def test_mixed_offsets_are_the_running_sum_of_record_sizes():
    # d = 64: records of kv 6 / 5 / 4 / 3 are 26 / 22 / 18 / 14 bytes
    cls = np.array([0, 3, 3, 1, 2, 0], dtype=np.uint8)
    off = oracle.mixed_offsets(64, (6, 5, 4, 3), cls)
    assert off.tolist() == [0, 26, 40, 54, 76, 94, 120]
    with pytest.raises(ValueError):
        oracle.mixed_offsets(64, (6, 5), cls)  # class 3 of only 2


def test_mixed_lookup_with_one_class_is_the_single_rate_lookup():
    d, kv, rows = 128, 5, 300
    recs = workload.random_records(rows, d, kv, seed=61)
    ids = np.random.default_rng(5).integers(-3, rows + 3, size=700)
    cls = np.zeros(rows, dtype=np.uint8)
    for raw in (False, True):
        exp, bad = oracle.lookup_decode(LUT, recs, rows, d, kv, ids, raw=raw)
        got, bad2 = oracle.lookup_decode_mixed(LUT, recs.reshape(-1), d, (kv,), cls, ids, raw=raw)
        assert bad == bad2 > 0
        assert (got == exp).all()


@pytest.mark.parametrize("d", [64, 256])
def test_mixed_lookup_reads_each_row_at_its_own_rate(d):
    # four single-rate tables; the mixed table takes row i from the table of
    # row i's class, so its lookups must equal those single-rate lookups
    rows = 400
    kvs = (6, 5, 4, 3)
    tables = [workload.random_records(rows, d, k, seed=70 + k) for k in kvs]
    cls = np.random.default_rng(9).integers(0, 4, size=rows).astype(np.uint8)
    packed = np.concatenate([tables[c][i] for i, c in enumerate(cls)])
    ids = np.random.default_rng(10).integers(0, rows, size=1000)
    got, bad = oracle.lookup_decode_mixed(LUT, packed, d, kvs, cls, ids)
    assert bad == 0
    for c, k in enumerate(kvs):
        sel = cls[ids] == c
        exp, _ = oracle.lookup_decode(LUT, tables[c], rows, d, k, ids[sel])
        assert (got[sel] == exp).all(), c
    # and the workload's packer lays the records out where the oracle reads them
    off = oracle.mixed_offsets(d, kvs, cls)
    assert (workload.mixed_layout(d, kvs, cls) == off).all()
    rec = workload.random_mixed_records(d, kvs, cls, seed=3)
    assert rec.size == int(off[-1])
    for i in (0, 1, rows - 1):
        R = workload.record_bytes(d, kvs[cls[i]])
        nb = R - 2
        a = int(rec[off[i] + nb]) | int(rec[off[i] + nb + 1]) << 8
        assert 0x3D00 <= a <= 0x4180, hex(a)  # a lognormal(0, 0.5) scale (e^-3.5 .. e^3.5)


def test_rank_classes_follow_access_rank():
    rows = 100_000
    cls = workload.rank_classes(rows, seed=202)
    assert np.bincount(cls, minlength=4).tolist() == [5_000, 15_000, 30_000, 50_000]
    ids = workload.zipf_ids(rows, 50_000, seed=202)
    share = np.bincount(cls[ids], minlength=4) / ids.size
    assert share[0] > 0.8 and share[3] < 0.05  # hot rows are the high-rate ones


# ---------------------------------------------------------------------------
# tie rule of the encoder, pinned by brute force over paths
# ---------------------------------------------------------------------------

def _window_costs(lut: np.ndarray, z: np.ndarray, T: int) -> list[np.ndarray]:
    """Branch cost of every 16-bit window at each step t, as the oracle forms
    it ((z0 - g0)^2 + (z1 - g1)^2 in fp64, g the signed codebook pair), from
    the hash written out here."""
    w = np.arange(1 << 16, dtype=np.int64)
    idx, neg = ((w * w + w) % (1 << 32) >> 7) & 511, (w >> 15) & 1
    g = lut.view(np.float16).astype(np.float64)[idx]
    g[neg == 1] *= -1.0
    return [(z[2 * t] - g[:, 0]) ** 2 + (z[2 * t + 1] - g[:, 1]) ** 2 for t in range(T)]


def _assert_exact(lut: np.ndarray, z: np.ndarray, costs: list[np.ndarray]) -> None:
    """The premise of the tie derivation: every cost is the exact value of
    its formula, a multiple of 2^-44 below 2^7, so every sum of four of them
    is exact in fp64 and "optimal" does not depend on the order of addition."""
    w = np.arange(1 << 16, dtype=np.int64)
    idx, neg = ((w * w + w) % (1 << 32) >> 7) & 511, (w >> 15) & 1
    g = lut.view(np.float16).astype(np.float64)[idx]
    g[neg == 1] *= -1.0
    for t, c in enumerate(costs):
        e0, e1 = z[2 * t] - g[:, 0], z[2 * t + 1] - g[:, 1]
        # differences and squares exact (few-bit z, fp16 g); the sum exact
        # when its rounding error (TwoSum) is zero
        assert ((e0 + g[:, 0]) == z[2 * t]).all() and ((e1 + g[:, 1]) == z[2 * t + 1]).all()
        a, b = e0 * e0, e1 * e1
        bb = c - a
        assert ((a - (c - bb)) + (b - bb) == 0).all()
        q = c * 2.0**44
        assert (q == np.floor(q)).all() and (c < 128).all()


def _free_start_sums(costs, order, chunk=1 << 22):
    """Yields (base, sums) over every free-start path b of 28 bits at d = 8,
    kv = 4: b's bits [4k, 4k + 16) are the window of the k-th visited step
    (bits 0..11 the start memory), sums[b - base] its cost."""
    for base in range(0, 1 << 28, chunk):
        b = np.arange(base, base + chunk, dtype=np.int64)
        tot = costs[order[0]][b & 0xFFFF]
        for k in range(1, 4):
            tot = tot + costs[order[k]][(b >> (4 * k)) & 0xFFFF]
        yield base, tot


def _tie_lut(kind: str) -> np.ndarray:
    """Codebooks under which many paths cost the same: "paired" makes
    entries 2j and 2j + 1 equal; "constant" gives every entry (1, -0.5), so
    a window's cost depends on its sign bit alone; "two-valued" gives even
    and odd entries two different pairs."""
    if kind == "gaussian":
        return LUT
    lut = LUT.copy()
    if kind == "paired":
        lut[1::2] = lut[0::2]
    elif kind == "constant":
        lut[:] = [0x3C00, 0xB800]
    else:
        lut[0::2] = [0x3C00, 0xB800]
        lut[1::2] = [0xBA00, 0x3E00]
    return lut


@pytest.mark.parametrize("lut_kind,z", [
    ("gaussian", np.zeros(8)),                      # every window ties with its complement
    ("paired", np.zeros(8)),
    ("constant", np.array([0.5, -1.25, 0, 0, 0, 0, 1.0, 0])),
    ("two-valued", np.array([2.0, 0, 0, 0.75, -1.0, 0, 0.25, 0.5])),
], ids=["gaussian-zero", "paired-zero", "constant-sparse", "two-valued"])
def test_encoder_tie_rule_matches_brute_force_over_paths(lut_kind, z):
    """The encoders keep, among equal path metrics, the smallest predecessor r
    (the oldest kv bits of the window) at each step, and the smallest end
    memory in the start-finding pass. With exact arithmetic every optimal
    path has optimal prefixes, so walking back from the end and taking the
    smallest r that stays optimal picks, among all optimal paths ending in
    that memory, the one whose r's read from the last step back are smallest
    in lexicographic order. At d = 8, kv = 4 a free-start path is a 28-bit
    string b whose k-th visited window is bits [4k, 4k + 16), so r_k = bits
    [4k, 4k + 4) and the end memory = bits [16, 28): that order is the order
    of b as an integer. So the start-finding pass picks the smallest b of
    least cost, and the code pass (start memory fixed: only the first step's
    4 bits are free) the smallest code of least cost. Derived here by
    enumeration, not by calling the encoder."""
    d, kv, T = 8, 4, 4
    lut = _tie_lut(lut_kind)
    costs = _window_costs(lut, z, T)
    _assert_exact(lut, z, costs)
    rot = T // 2
    order = [(k + rot) % T for k in range(T)]
    best, best_b = np.inf, None
    ties = 0
    for base, tot in _free_start_sums(costs, order):
        m = tot.min()
        if m < best:
            best, best_b, ties = m, base + int(np.argmax(tot == m)), int((tot == m).sum())
        elif m == best:
            ties += int((tot == m).sum())
    # memory before step 0 = after the visited step T - rot - 1 (step T - 1)
    k = T - rot - 1
    w_h = (best_b >> (4 * k + 4)) & 0xFFF
    # code pass: codes whose last 12 bits are w_h; windows of the closed path
    # b' = w_h | code << 12 in natural step order
    cand = np.arange(16, dtype=np.int64) | (w_h << 4)
    bp = (cand >> 4) | (cand << 12)
    tot = sum(costs[t][(bp >> (4 * t)) & 0xFFFF] for t in range(T))
    code = int(cand[int(np.argmax(tot == tot.min()))])
    # the case has ties for the rule to decide
    assert ties > 1
    heur = oracle.tcq_encode(z, d, kv, lut, oracle.ENC_HEURISTIC)
    assert _code_int(heur.code) == code
    assert heur.cost == tot.min()

    # exact mode: the heuristic's code is the incumbent and a start replaces
    # it only when strictly better; starts are tried by increasing free-start
    # bound, then by memory
    allc = np.arange(1 << 16, dtype=np.int64)
    ball = (allc >> 4) | (allc << 12)
    closed = sum(costs[t][(ball >> (4 * t)) & 0xFFFF] for t in range(T))
    gmin = closed.min()
    exact = oracle.tcq_encode(z, d, kv, lut, oracle.ENC_EXACT)
    assert exact.cost == gmin
    if tot.min() == gmin:
        assert _code_int(exact.code) == code
    else:
        F = np.full(1 << 12, np.inf)
        for base, s_ in _free_start_sums(costs, list(range(T))):
            ends = (np.arange(base, base + s_.size, dtype=np.int64) >> 16)
            np.minimum.at(F, ends, s_)
        starts = sorted(range(1 << 12), key=lambda w: (F[w], w))
        first = next(w for w in starts if (closed[(allc >> 4) == w] == gmin).any())
        sel = np.nonzero(((allc >> 4) == first) & (closed == gmin))[0]
        assert _code_int(exact.code) == int(sel.min())


# ---------------------------------------------------------------------------
# the scaled output for tiny products, against exact rational arithmetic
# ---------------------------------------------------------------------------

def _bf16_rne_exact(q: Fraction) -> int:
    """bf16 bits of the rational q rounded to nearest, ties to even, worked
    out on the bf16 grid itself (spacing 2^(E-7) in binade E, 2^-133 below
    2^-126)."""
    sgn = 0x8000 if q < 0 else 0
    a = abs(q)
    if a == 0:
        return sgn
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    E = max(E, -126)
    unit = Fraction(2) ** (E - 7)
    k, rem = divmod(a, unit)
    k = int(k)
    if rem * 2 > unit or (rem * 2 == unit and k % 2 == 1):
        k += 1
    bits = ((E + 127) << 7) + (k - 128)
    return sgn | min(bits, 0x7F80)


def _fp16_fraction(h: int) -> Fraction:
    e, m = (h >> 10) & 31, h & 1023
    v = Fraction(m, 1 << 24) if e == 0 else Fraction(1024 + m) * Fraction(2) ** (e - 25)
    return -v if h & 0x8000 else v


def _bf16_fraction(b: int) -> Fraction:
    e, m = (b >> 7) & 255, b & 127
    v = Fraction(m) * Fraction(2) ** -133 if e == 0 else Fraction(128 + m) * Fraction(2) ** (e - 134)
    return -v if b & 0x8000 else v


def test_scaled_row_of_tiny_products_is_the_single_rounding_of_the_exact_product():
    # decode_record against exact rationals where the product alpha * f falls
    # below 2^-126 (bf16 subnormals) or near it: no intermediate fp32 rounding
    rng = np.random.default_rng(77)
    lut = rng.integers(0, 0x7BFF, size=1024, dtype=np.uint16)
    lut[::7] = rng.integers(0, 0x0400, size=lut[::7].size, dtype=np.uint16)  # fp16 subnormals
    lut[::5] |= 0x8000
    lut[:4] = [0x0000, 0x8000, 0x0001, 0x03FF]
    lut = lut.reshape(512, 2)
    d, kv = 64, 4
    nb = kv * d // 16
    alphas = [0x0001, 0x8001, 0x007F, 0x0080, 0x00FF, 0x0100, 0x0C7F, 0x0C00, 0x0880, 0x0455]
    checked = 0
    for ab in alphas:
        rec = np.empty(nb + 2, dtype=np.uint8)
        rec[:nb] = rng.integers(0, 256, size=nb, dtype=np.uint8)
        rec[nb], rec[nb + 1] = ab & 0xFF, ab >> 8
        f = oracle.decode_code(lut, rec[:nb], d, kv)
        y = oracle.decode_record(lut, rec, d, kv)
        a = _bf16_fraction(ab)
        for fi, yi in zip(f, y):
            assert int(yi) == _bf16_rne_exact(a * _fp16_fraction(int(fi))), (hex(ab), hex(int(fi)))
            checked += 1
    assert checked == len(alphas) * d


def test_bf16_rounding_of_subnormal_products_against_exact_rationals():
    # every bf16 scale with a small exponent field times random fp16 values:
    # the oracle's one-step rounding equals the exact rational rounding; also
    # products that lie just below a midpoint of the bf16 subnormal grid
    # (closer than fp32's spacing there), where rounding through fp32 first
    # would end 1 ulp off
    near_mid_bf16 = [0x00B9, 0x00CF, 0x0139, 0x014F, 0x01B9, 0x01CF, 0x0239, 0x024F, 0x02B9, 0x02CF,
                     0x0339, 0x034F, 0x03CF, 0x044F, 0x80B9, 0x80CF, 0x8139, 0x814F, 0x81B9, 0x81CF,
                     0x8239, 0x824F, 0x82B9, 0x82CF, 0x8339, 0x834F, 0x83CF, 0x844F]
    near_mid_fp16 = [0x0589, 0x062F, 0x0989, 0x0A2F, 0x0D89, 0x0E2F, 0x1189, 0x122F, 0x1589, 0x162F,
                     0x1989, 0x1A2F, 0x1E2F, 0x222F, 0x8589, 0x862F, 0x8989, 0x8A2F, 0x8D89, 0x8E2F,
                     0x9189, 0x922F, 0x9589, 0x962F, 0x9989, 0x9A2F, 0x9E2F, 0xA22F]
    for ab in near_mid_bf16:
        for h in near_mid_fp16:
            q = _bf16_fraction(ab) * _fp16_fraction(h)
            assert oracle.bf16_from_double(float(q)) == _bf16_rne_exact(q), (hex(ab), hex(h))
    rng = np.random.default_rng(78)
    for ab in list(range(0, 0x1000, 37)) + [0x0001, 0x007F, 0x0080, 0x0C7F, 0x0C80]:
        for h in rng.integers(0, 0x7C00, size=24):
            q = _bf16_fraction(ab) * _fp16_fraction(int(h))
            assert oracle.bf16_from_double(float(q)) == _bf16_rne_exact(q), (hex(ab), hex(int(h)))


# ---------------------------------------------------------------------------
# rows whose norm is not finite
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_rows_with_non_finite_norm_encode_to_the_zero_record(bad):
    # z = sqrt(d) e / ||e|| and alpha = ||e|| / ||f(c)|| need a finite nonzero
    # norm; a row holding an inf or a NaN is stored like a zero row
    d, kv = 64, 4
    e = workload.gaussian_rows(1, d, seed=31)[0]
    e[5] = bad
    rec, _, alpha = oracle.encode_row(e, d, kv, LUT, oracle.ENC_HEURISTIC)
    assert alpha == 0.0 and (rec == 0).all()
    recs, _ = oracle.encode_rows(e[None, :], d, kv, LUT, oracle.ENC_HEURISTIC)
    assert (recs == 0).all()


def test_shard_plan_is_a_stable_grouping_by_owner():
    """The oracle's shard plan against a construction by hand: walk the
    shards in order and, within each, the batch in order."""
    rng = np.random.default_rng(4100)
    for trial in range(60):
        shards = int(rng.integers(1, 9))
        rps = int(rng.integers(1, 50))
        n = int(rng.integers(0, 300))
        ids = rng.integers(-5, shards * rps + 10, n).astype(np.int64)
        local_ids, positions, counts = oracle.shard_plan(ids, rps, shards)
        exp_local, exp_pos, exp_counts = [], [-1] * n, []
        for s in range(shards):
            mine = [j for j in range(n) if 0 <= ids[j] < shards * rps and ids[j] // rps == s]
            exp_counts.append(len(mine))
            for j in mine:
                exp_pos[j] = len(exp_local)
                exp_local.append(int(ids[j]) - s * rps)
        assert local_ids.tolist() == exp_local
        assert positions.tolist() == exp_pos
        assert counts.tolist() == exp_counts


def test_gather_records_copies_rows_and_zeroes_bad_ids():
    rng = np.random.default_rng(4101)
    recs = rng.integers(0, 256, (37, 18), dtype=np.uint8)
    ids = np.array([3, 36, 0, -1, 37, 3, 2**40], dtype=np.int64)
    got = oracle.gather_records(recs, 37, ids)
    for k, i in enumerate(ids):
        assert (got[k] == (recs[i] if 0 <= i < 37 else 0)).all()
