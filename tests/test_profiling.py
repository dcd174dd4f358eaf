"""Host checks of the rocprofv3 helpers behind bench.py's roofline traffic."""
import csv
import json
import os

from linear_cross_entropy_ce_amd import profiling as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CFG = "INS_3CfgINS_9TileShapeILi256ELi256ELi64ELi2ELi4EEEDF16bEE"
_DEM = "fce::Cfg<fce::TileShape<256, 256, 64, 2, 4>, __bf16>"
MANGLED = {
    # k_bwd_grad<C, A_KMAJOR, FILTER>: the first flag tells dW from dX
    f"_ZN3fce12_GLOBAL__N_110k_bwd_grad{_CFG}Lb0ELb0EEEvNS0_8GradArgsINT_4ElemEEE": "bwd_dw",
    f"_ZN3fce12_GLOBAL__N_110k_bwd_grad{_CFG}Lb0ELb1EEEvNS0_8GradArgsINT_4ElemEEE": "bwd_dw",
    f"_ZN3fce12_GLOBAL__N_110k_bwd_grad{_CFG}Lb1ELb0EEEvNS0_8GradArgsINT_4ElemEEE": "bwd_dx",
    f"_ZN3fce12_GLOBAL__N_110k_bwd_grad{_CFG}Lb1ELb1EEEvNS0_8GradArgsINT_4ElemEEE": "bwd_dx",
    f"void fce::(anonymous namespace)::k_bwd_grad<{_DEM}, true, false>(GradArgs<__bf16>)": "bwd_dx",
    f"void fce::(anonymous namespace)::k_bwd_grad<{_DEM}, false, true>(GradArgs<__bf16>)": "bwd_dw",
    f"_ZN3fce12_GLOBAL__N_18k_bwd_dz{_CFG}Lb1ELb0EEEvNS0_6DzArgsINT_4ElemEEE": "bwd_dz",
    # k_bwd_grad_pair<C, DW_KMAJOR, DW_TRANS>: dW and dX of a block in one grid
    f"_ZN3fce12_GLOBAL__N_115k_bwd_grad_pair{_CFG}Lb1ELb1EEEvNS0_8GradArgsIDF16bEES7_iii": "bwd_grad",
    f"void fce::(anonymous namespace)::k_bwd_grad_pair<{_DEM}, false, false>(GradArgs<__bf16>, GradArgs<__bf16>, int, int, int)": "bwd_grad",
    # the filtered products of a block in one grid
    f"_ZN3fce12_GLOBAL__N_120k_bwd_grad_pair_filt{_CFG}EEvNS0_8GradArgsIDF16bEES7_S7_iiii": "bwd_grad",
    # k_fwd_lse<C, SMOOTH, STORE>: the storing one belongs to store-logits
    f"_ZN3fce12_GLOBAL__N_19k_fwd_lse{_CFG}Lb1ELb0EEEvNS0_7FwdArgsINT_4ElemEEE": "fwd_lse",
    f"_ZN3fce12_GLOBAL__N_19k_fwd_lse{_CFG}Lb0ELb1EEEvNS0_7FwdArgsINT_4ElemEEE": "sl_fwd",
    "_ZN3fce12_GLOBAL__N_111k_ce_logitsIDF16bLb0EEEvNS0_6CeArgsE": "ce_logits",
    "fce::(anonymous namespace)::k_dx_reduce(float const*, int, long)": "dx_reduce",
    "fce::(anonymous namespace)::k_lse_merge(float __vector(4) const*, int, long)": "lse_merge",
    "__amd_rocclr_copyBuffer": None,
}


def test_kernel_names_map_to_timer_names():
    for name, key in MANGLED.items():
        assert P.kernel_key(name) == key, name


def _write_counters(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_traffic_scales_by_copy_calibration(tmp_path):
    dz = [k for k, v in MANGLED.items() if v == "bwd_dz"][0]
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    # a counter reported in two parts for one dispatch is summed
    _write_counters(tmp_path / "f.csv", [(1, dz, "FETCH_SIZE", 100.0), (1, dz, "FETCH_SIZE", 50.0),
                                         (2, dz, "FETCH_SIZE", 250.0)])
    _write_counters(tmp_path / "w.csv", [(1, dz, "WRITE_SIZE", 64.0), (2, dz, "WRITE_SIZE", 64.0)])
    _write_counters(tmp_path / "cf.csv", [(7, neg, "FETCH_SIZE", 512.0)])  # half of 1 MiB
    _write_counters(tmp_path / "cw.csv", [(7, neg, "WRITE_SIZE", 1024.0)])
    out = tmp_path / "prof"
    P.main(["traffic", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
            "--copy-fetch", str(tmp_path / "cf.csv"), "--copy-write", str(tmp_path / "cw.csv"),
            "--copy-mib", "1", "--workload", "w", "--out", str(out)])
    rec = json.load(open(out / "bwd_dz_w_traffic.json"))
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["dispatches"] == 2
    # (150 + 250) / 2 KiB fetched x 2, plus 64 KiB written
    assert rec["hbm_bytes_per_launch"] == 200 * 1024 * 2 + 64 * 1024
    assert rec["source_sha256"] == P.source_digest()


def test_committed_traffic_records_are_consistent():
    prof = os.path.join(ROOT, "profiles")
    recs = [json.load(open(os.path.join(prof, f))) for f in os.listdir(prof)
            if f.endswith("_traffic.json")]
    assert recs, "no traffic records under profiles/"
    for r in recs:
        hbm = (r["fetch_kib_per_dispatch"] * r["fetch_factor"]
               + r["write_kib_per_dispatch"] * r["write_factor"]) * 1024
        assert abs(hbm - r["hbm_bytes_per_launch"]) <= 1, r["kernel"]
        assert r["commands"], r["kernel"]
