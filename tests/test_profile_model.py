"""Host logic of the counter summaries: the tile-walk request model and the kernel-name parsing."""
import itertools

import pytest

from exact_attention_forward_amd import profile as P


def brute_prefix(N, br, bc):
    # every key block a causal query tile walks: blocks whose first key is <= the tile's last row
    total = 0
    for t in range(-(-N // br)):
        last = min((t + 1) * br, N) - 1
        total += sum(bc for j0 in range(0, N, bc) if j0 <= last)
    return total


def brute_suffix(N, bk, bq):
    # every query block a causal key tile walks: blocks whose last row reaches the tile's first key
    total = 0
    for t in range(-(-N // bk)):
        first = t * bk
        total += sum(bq for q0 in range(0, N, bq) if q0 + bq - 1 >= first)
    return total


@pytest.mark.parametrize("N,a,b", list(itertools.product([1, 31, 64, 300, 1024], [64, 128], [32, 64])))
def test_walk_counts_match_enumeration(N, a, b):
    assert P.prefix_keys(N, a, b) == brute_prefix(N, a, b)
    assert P.suffix_rows(N, a, b) == brute_suffix(N, a, b)


def test_bf16_forward_requests_match_closed_form():
    # causal forward at B64 H16 T1024 hd64, 128-row query tiles: per head Nd + (G+1) N d elements
    # are read (Q once, the K and V prefix of G = 8 tiles), 2 bytes each
    m = P.kernel_model("C3", "fwd32_kernel")
    N, d, G, heads = 1024, 64, 8, 64 * 16
    assert m["req_read"] == (N * d + (G + 1) * N * d) * 2 * heads
    assert m["comp_read"] == 3 * N * d * 2 * heads
    assert m["write"] == (4 * N * d + 4 * N) * heads


def test_kernel_names_map_to_workloads():
    assert P.workload_of("void fa::fwd32_kernel<fa::bf16_t, 64, true, 0, 2, 32, 2>(fa::FwdArgs)") == "C3"
    assert P.workload_of("void fa::fwd64_kernel<fa::bf16_t, true, 0>(fa::FwdArgs)") == "C3"
    assert P.workload_of("void fa::dkv64_kernel<fa::bf16_t, true, 1>(fa::BwdArgs)") == "C3"
    assert P.workload_of("void fa::dkv64_kernel<fa::f16_t, true, 0>(fa::BwdArgs)") is None
    assert P.family("void fa::dkv64_kernel<fa::bf16_t, true, 0>(fa::BwdArgs)") == "dkv64_kernel"
    assert P.stage_of("dkv64_kernel") == "dkv" and P.stage_of("dq32_kernel") == "dq"
    assert P.compulsory_bytes("fwd64_kernel", 64, 16, 1024, 64, 2, True) == \
        P.compulsory_bytes("fwd32_kernel", 64, 16, 1024, 64, 2, True)
    assert P.workload_of("void fa::dkv32_kernel<fa::bf16_t, 128, true, 1, 4, 64>(fa::BwdArgs)") == "C4"
    assert P.workload_of("void fa::dq32_kernel<fa::f16_t, 64, true, 0, 4, 64, true>(fa::BwdArgs)") is None
    assert P.workload_of("void fa::dq_kernel<float, 64, true, 0, 4, 2, 32, false>(fa::BwdArgs)") == "C2"
    assert P.workload_of("__amd_rocclr_copyBuffer") is None
    assert P.family("void fa::delta_kernel<float, 64>(fa::BwdArgs)") == "delta_kernel"


def test_split_report_table(tmp_path):
    """The split summary has one row per workload, one column per split count, and picks the fastest split."""
    import json

    from exact_attention_forward_amd import profile

    row = {"workload": "w", "B": 1, "H": 4, "T": 8192, "hd": 128, "dtype": "bf16", "causal": True, "precision": 1,
           "plain_ms": 0.23, "plain_tflops": 600.0,
           "splits": [{"nsplit": 2, "ms": 0.2, "speedup": 1.15, "tflops": 690.0, "max_abs_diff_O": 1e-4,
                       "max_abs_diff_L": 2e-6},
                      {"nsplit": 4, "ms": 0.18, "speedup": 1.28, "tflops": 766.0, "max_abs_diff_O": 3e-4,
                       "max_abs_diff_L": 1e-6}]}
    log = tmp_path / "split.log"
    log.write_text(json.dumps(row) + "\n" + json.dumps({"split_workloads": 1, "device": "d", "arch": "gfx950",
                                                        "cus": 256, "hip": "7"}) + "\n")
    out = tmp_path / "split.md"
    profile.split_report(str(log), str(out))
    text = out.read_text()
    table = [l for l in text.splitlines() if l.startswith("| B1 H4")]
    assert len(table) == 1
    assert "2 splits | 4 splits" in text
    assert "766.0 (4 splits)" in table[0] and "3.00e-04" in table[0] and "2.00e-06" in table[0]


# Each tensor of the backward interface with its element count per head (T rows
# of hd values, or T scalars) and whether it is an input of dtype e or float32.
def _inventory(T, hd, e):
    rows = T * hd
    return {"q": rows * e, "k": rows * e, "v": rows * e, "dO": rows * e, "O": rows * 4, "L": T * 4, "D": T * 4,
            "dQ": rows * 4, "dK": rows * 4, "dV": rows * 4}


# What each kernel reads and writes, tensor by tensor.
_ROLES = {
    "fwd32_kernel": (("q", "k", "v"), ("O", "L")),
    "dq32_kernel": (("q", "k", "v", "dO", "L", "D"), ("dQ",)),
    "dq32_kernel+D": (("q", "k", "v", "dO", "L", "O"), ("dQ", "D")),
    "dkv32_kernel": (("q", "k", "v", "dO", "L", "D"), ("dK", "dV")),
    "delta_kernel": (("O", "dO"), ("D",)),
}


@pytest.mark.parametrize("shape", [(64, 16, 1024, 64, 2), (64, 16, 1024, 64, 4), (4, 16, 8192, 128, 2),
                                   (2, 3, 300, 32, 4)])
@pytest.mark.parametrize("kernel", sorted(_ROLES))
def test_compulsory_bytes_count_each_tensor_once(shape, kernel):
    B, H, T, hd, e = shape
    inv = _inventory(T, hd, e)
    reads, writes = _ROLES[kernel]
    fam, fused = kernel.split("+")[0], kernel.endswith("+D")
    r, w = P.compulsory_bytes(fam, B, H, T, hd, e, fused_d=fused)
    assert r == B * H * sum(inv[t] for t in reads)
    assert w == B * H * sum(inv[t] for t in writes)


def test_compulsory_bytes_match_the_gpt2_medium_figures():
    # B64 H16 T1024 hd64 bf16: forward 0.675 GB; backward D pre-pass 0.407, dQ 0.814 and dK/dV 1.082 GB
    gb = lambda fam, fused=False: sum(P.compulsory_bytes(fam, 64, 16, 1024, 64, 2, fused)) / 1e9
    assert round(gb("fwd32_kernel"), 3) == 0.675
    assert round(gb("delta_kernel"), 3) == 0.407
    assert round(gb("dq32_kernel"), 3) == 0.814
    assert round(gb("dkv32_kernel"), 3) == 1.082
    # D fused into the dQ kernel: the pre-pass's second read of dO and the dQ kernel's read of D disappear
    n, r = 64 * 16 * 1024 * 64, 64 * 16 * 1024
    assert gb("dq32_kernel", True) == pytest.approx(gb("dq32_kernel") + gb("delta_kernel") - (2 * n + 4 * r) / 1e9)
    assert P.kernel_model("C3", "dq32_kernel")["comp_read"] == P.compulsory_bytes("dq32_kernel", 64, 16, 1024, 64, 2,
                                                                                  True)[0]
