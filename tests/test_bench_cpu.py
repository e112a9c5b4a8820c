"""Host-side logic of bench.py (no GPU): the algorithmic byte counts the metric divides by, and
the refusal to run on more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import moe_synth as ms  # noqa: E402

# Compulsory megabytes per decode layer (dispatch, combine, total), computed stage by stage from
# the staged method's reads and writes with a 4-byte metadata word per row: route NT*E*4 + NT*R*8;
# send NT*P + M*(P + 4) + 8*NT*R; network 2*M*(P + 4); unpack 2*M*(P + 4) + 8*M; combine
# shuffle 2*M*Pc + 4*M; network back 2*M*Pc; weighted sum M*Pc + 8*NT*R + NT*Pc (NT = N*T,
# M = NT*R, P the dispatched row, Pc = 2H).  The library's rows carry an 8-byte metadata pair and
# its calls also read the small offset tables, so its counts sit slightly above these.
PUBLISHED_MB = {  # as printed: rounded to the digits shown
    "tiny": ("0.18", "0.18", "0.37"),
    "mixtral_8x7b_decode": ("92.4", "92.3", "185"),
    "deepseek_v3_decode": ("2413", "2408", "4821"),
    "deepseek_v3_decode_fp8": ("1247", "2408", "3655"),
    "qwen3_235b_prefill": ("5517", "5504", "11022"),
    "kimi_k2_worst": ("2498", "4816", "7314"),
}


@pytest.mark.parametrize("name", sorted(PUBLISHED_MB))
def test_algorithmic_bytes_match_the_stage_counts(name):
    c = ms.CONFIGS[name]
    ab = bench.alg_bytes(c)
    dispatch = ab["route"] + ab["dispatch_send"] + ab["net_dispatch"] + ab["dispatch_recv"]
    want_d, want_c, want_t = PUBLISHED_MB[name]
    for got, printed in ((dispatch, want_d), (ab["combine"], want_c), (ab["total"], want_t)):
        got_mb, want = got / 1e6, float(printed)
        half_digit = 0.5 * 10.0 ** -(len(printed.split(".")[1]) if "." in printed else 0)
        # the printed count within its rounding, plus at most 0.1% for the wider metadata
        assert want - half_digit <= got_mb <= want + half_digit + 1e-3 * want, (name, got_mb, printed)
    assert ab["total"] == dispatch + ab["combine"]


def test_token_counts_scale_the_bytes():
    # absent tokens are neither read nor written: the ragged mix counts only its present tokens
    full = bench.alg_bytes(ms.CONFIGS["deepseek_v3_decode"])["total"]
    c = ms.CONFIGS["deepseek_v3_decode_ragged"]
    tok = ms.config_tokens(c)
    ragged = bench.alg_bytes(c)["total"]
    frac = float(tok.sum()) / (c.N * c.T)
    assert abs(ragged / full - frac) < 0.01


def test_memory_side_cache_rule():
    # the exchanged rows of e4m3 DeepSeek-V3 (242 MB) fit in the 256 MB cache; bf16 (470 MB) and
    # Kimi-K2 (485 MB) do not
    assert bench.exchange_fits_mall(ms.CONFIGS["deepseek_v3_decode_fp8"])
    assert not bench.exchange_fits_mall(ms.CONFIGS["deepseek_v3_decode"])
    assert not bench.exchange_fits_mall(ms.CONFIGS["kimi_k2_worst"])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_leg_on_the_tiny_workload():
    # the oracle leg runs without a GPU: its contract fields, the per-stage times that make up the
    # layer, and the threaded run's output equal to the single-threaded one (checked inside)
    r = bench.cpu_baseline("tiny", budget_s=1.0)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["cores"] == 1 and r["value"] > 0
    assert set(r["per_stage_us"]) == {"route", "dispatch_send", "net_dispatch", "dispatch_recv", "combine"}
    assert r["threaded"]["cores"] >= 1 and r["threaded"]["value"] > 0
    assert "tiny" in r["sample"]
