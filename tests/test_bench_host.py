"""Host logic of bench.py (no GPU): the refusal of several GPUs, the algorithmic byte and
work models, the timing statistics and the parsing of the committed profile summaries."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402

N = 1 << 16
LIMB = N * 4


def test_several_gpus_are_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_headline_call():
    # batch 8 at level 36: ciphertexts in (8 x 2 x 36 limbs) and out (the same), and the
    # key's b rows once (3 digits x 48 primes); the stored variant reads the a rows too
    ct = 8 * 2 * 36 * LIMB
    key_half = 3 * 48 * LIMB
    assert bench.hbm_bytes(36, 8, True) == 2 * ct + key_half
    assert bench.hbm_bytes(36, 8, False) == 2 * ct + 2 * key_half
    assert round(bench.hbm_bytes(36, 8, True) / 1e6, 1) == 339.7
    # partial last digit at level 13 (digits of 12 and 1 primes): two digits of key rows
    assert bench.hbm_bytes(13, 1, True) == 2 * (2 * 13 * LIMB) + 2 * (13 + 12) * LIMB
    # hoisting: one ciphertext in, one output per key, every key's rows
    assert bench.hbm_bytes(36, 1, True, 16) == 2 * 36 * LIMB + 16 * 2 * 36 * LIMB + 16 * key_half


def _units(monkeypatch, **costs):
    slots = {k: 0 for k in bench.SLOT}
    slots.update(costs)
    monkeypatch.setattr(bench, "SLOT", slots)
    return bench.work_model(36, 1, True)


def test_work_model_counts_the_method_once(monkeypatch):
    # one switch at level 36 (dnum 3, alpha 12, K 12): 240 limb transforms of N/2 * 16
    # butterflies each, sum_j alpha_j (E - alpha_j) N + 2 K l N conversion MACs,
    # 2 d E N inner-product MACs and d E N (1 + rejection) ChaCha words
    # the end of ModDown's four word operations per coefficient and limb ((x - conv) * P^-1 +
    # sigma(c0) on both halves, beyond its constant multiplies) are priced directly
    base = _units(monkeypatch)
    assert sum(base.values()) == 4 * N * 36
    bfly = sum(_units(monkeypatch, bfly=1).values()) - sum(base.values())
    assert bfly == 240 * (N // 2) * 16
    mac = _units(monkeypatch, mac=1)
    assert mac["modup_conv"] + mac["moddown_conv"] == (3 * 12 * 36 + 2 * 12 * 36) * N
    assert mac["ip_special"] + mac["ip_final"] - base["ip_final"] == 2 * 3 * 48 * N
    words = sum(_units(monkeypatch, chacha_word=1).values()) - sum(base.values())
    assert words == pytest.approx(3 * 48 * N * 1.0075)
    monkeypatch.undo()
    stored, regen = bench.work_model(36, 1, False), bench.work_model(36, 1, True)
    assert regen["row"] == stored["row"] and regen["ip_final"] > stored["ip_final"]


def test_batch_shares_the_regenerated_key():
    # the a-half of a shared key is regenerated once per call, not once per ciphertext
    one, eight = bench.work_model(36, 1, True), bench.work_model(36, 8, True)
    s1, s8 = bench.work_model(36, 1, False), bench.work_model(36, 8, False)
    assert (eight["ip_final"] - s8["ip_final"]) == pytest.approx(one["ip_final"] - s1["ip_final"])
    assert s8["modup_conv"] == 8 * s1["modup_conv"]


def test_timing_statistics():
    samples = [1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0, 9.0, 10.0, 11.0]
    st = bench.stats(samples, [6.0], 8, "key_switches_per_s")
    assert st["ms_median"] == 6.0
    assert st["ms_p10"] == 2.0 and st["ms_p90"] == 10.0
    assert st["ms_per_call"] == 6.0
    assert st["key_switches_per_s"] == pytest.approx(8 / 6e-3, abs=0.1)
    assert st["calls_timed"] == 11


def test_profile_summaries_are_quoted_only_for_the_sources_they_were_taken_on(monkeypatch):
    if bench._current_profile("valu_issue_keyswitch_batch8_l36.md") is not None:
        issue = bench.read_issue("ip_final")
        assert issue and 3.5 < issue["cycles_per_valu_inst"] < 8 and 0 < issue["issue_frac"] <= 1.2
        traffic = bench.read_traffic("ip_final")
        assert traffic and traffic["fetch_bytes"] > 0 and traffic["write_bytes"] > 0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.read_issue("ip_final") is None
    assert bench.read_traffic("ip_final") is None


def test_instruction_rates_parse():
    rates = bench.read_valu_rates()
    assert rates is not None
    assert 30 < rates["v_mul_lo_u32"] < 45 and 55 < rates["v_add_u32"] < 75
    assert 3 < rates["butterfly"] < 5


def test_ntt_roofline_units():
    # a forward limb-NTT at N = 2^16: 2^15 * 16 butterflies, 512 KiB read and written once
    r = bench.ntt_roofline(1e6, 16, False, {"butterfly": 4.0})
    assert r["slots_per_limb"] == (N // 2) * 16 * bench.SLOT["bfly"]
    assert r["bytes_per_limb"] == 2 * LIMB
    assert r["valu_frac"] == pytest.approx(1e6 * r["slots_per_limb"] / bench.VALU_PEAK, abs=1e-4)
    assert r["hbm_frac"] == pytest.approx(1e6 * 2 * LIMB / 8e12, abs=1e-4)
    assert r["frac_vs_butterfly_rate"] == pytest.approx(1e6 * (N // 2) * 16 / 4e12, abs=1e-4)
    assert r["bound"] == "alu"
    # the inverse also scales by N^-1: one constant multiply per coefficient
    inv = bench.ntt_roofline(1e6, 16, True, None)
    assert inv["slots_per_limb"] - r["slots_per_limb"] == N * bench.SLOT["cmul"]
    assert "frac_vs_butterfly_rate" not in inv


def test_source_hash_follows_code_not_comments():
    paths = [os.path.join(ROOT, "rns_ckks_key_amd", "csrc", f) for f in ("kernels.hip", "modarith.h", "ckks_internal.h")]
    texts = [open(p).read() for p in paths]
    h = bench.kernel_source_hash(texts)
    assert h == bench.kernel_source_hash()
    commented = ["// a note\n" + texts[0].replace("\n", "  \n", 3) + "/* more */", texts[1], texts[2]]
    assert bench.kernel_source_hash(commented) == h
    changed = [texts[0] + "\nstatic int extra_symbol;", texts[1], texts[2]]
    assert bench.kernel_source_hash(changed) != h


def test_parity_gate_compares_every_oracle_output_with_every_variant():
    import numpy as np

    rng = np.random.default_rng(7)
    gpu = rng.integers(0, 2**32, (3, 2, 2, 8), dtype=np.uint64).astype(np.uint32)
    gpu_out = {"regen": gpu.copy(), "stored": gpu.copy()}
    oracle = [(0, "regen", gpu[0].astype(np.uint64)), (2, "stored", gpu[2].astype(np.uint64)),
              (0, "stored", gpu[0].astype(np.uint64))]
    p = bench.parity_check(gpu_out, oracle)
    assert p["bit_exact"] is True and p["ciphertexts"] == [0, 2] and p["outputs_compared"] == 6
    gpu_out["stored"][2, 1, 0, 5] ^= 1  # one residue of one variant
    p = bench.parity_check(gpu_out, oracle)
    assert p["bit_exact"] is False
    assert p["mismatches"] == [{"ciphertext": 2, "gpu_variant": "stored", "oracle_key": "stored"}]
    assert bench.parity_check(gpu_out, [])["bit_exact"] is False  # nothing compared proves nothing
