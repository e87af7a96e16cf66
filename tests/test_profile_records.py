"""Host logic of the profile records: kernel-name shortening, the traffic
record round trip and the source digest that invalidates stale records."""
import os

import bench
from sparse_attention_scores_amd import profile_summary as ps


def test_short_name_keeps_templates_drops_arguments():
    n = "void dsa::topk_rows_kernel<1024, 16384, 0, 2>(float const*, int, int*) [clone .kd]"
    assert ps.short_name(n) == "dsa::topk_rows_kernel<1024, 16384, 0, 2> [clone .kd]"
    assert ps.short_name("dsa::attend_gather_kernel(unsigned short const*)") == "dsa::attend_gather_kernel"


def test_traffic_record_round_trip(tmp_path):
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    hdr = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
    fetch.write_text(hdr + "1,probe_copy_kernel(uint4 const*),FETCH_SIZE,512\n"
                     "2,dsa::attend_gather_kernel(int),FETCH_SIZE,100\n"
                     "2,dsa::attend_gather_kernel(int),FETCH_SIZE,20\n"
                     "3,dsa::attend_gather_kernel(int),FETCH_SIZE,120\n")
    write.write_text(hdr + "1,probe_copy_kernel(uint4 const*),WRITE_SIZE,1024\n"
                     "2,dsa::attend_gather_kernel(int),WRITE_SIZE,8\n"
                     "3,dsa::attend_gather_kernel(int),WRITE_SIZE,8\n")
    text = ps.traffic(str(fetch), str(write), 1 << 20, "cmd f", "cmd w")
    rec = tmp_path / "r.txt"
    rec.write_text(text)
    digest, ff, wf, kern = ps.read_traffic(str(rec))
    assert digest == ps.source_digest()
    assert abs(ff - 2.0) < 1e-9 and abs(wf - 1.0) < 1e-9
    # per-dispatch averages: fetch (120 + 120) / 2, write 8
    assert kern == {"dsa::attend_gather_kernel": (120.0, 8.0)}


def test_bench_uses_record_only_for_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    name = f"dsa_step_{bench.WORKLOAD_NAME[2]}_hbm_traffic.txt"
    body = ("fetch_factor 2.0\nwrite_factor 1.0\n"
            "kernel dsa::attend_gather_kernel fetch_kib 10.0 write_kib 1.0 dispatches 2\n"
            "kernel dsa::attend_combine_kernel fetch_kib 4.0 write_kib 2.0 dispatches 2\n"
            "kernel dsa::index_scores_mfma_kernel<128,1,1,1,false> fetch_kib 7.0 write_kib 0.0 dispatches 2\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (prof / name).write_text(f"source_digest {ps.source_digest()}\n" + body)
    t, src = bench.measured_traffic(2, "attend")
    assert t == round((10 * 2 + 1 + 4 * 2 + 2) * 1024) and src.endswith(name)
    (prof / name).write_text("source_digest 0000\n" + body)
    assert bench.measured_traffic(2, "attend")[0] is None
    os.remove(prof / name)
    assert bench.measured_traffic(2, "attend") == (None, None)


def test_mfma_record_use_fraction(tmp_path):
    counters = tmp_path / "c.csv"
    stats = tmp_path / "s.csv"
    counters.write_text("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
                        "1,dsa::attend_gather_kernel(int),SQ_INSTS_MFMA,1000\n"
                        "1,dsa::attend_gather_kernel(int),SQ_VALU_MFMA_BUSY_CYCLES,1228800\n"
                        "2,dsa::attend_gather_kernel(int),SQ_INSTS_MFMA,1000\n"
                        "2,dsa::attend_gather_kernel(int),SQ_VALU_MFMA_BUSY_CYCLES,1228800\n"
                        "3,dsa::topk_seg_kernel<1024,16384>(float),SQ_VALU_MFMA_BUSY_CYCLES,0\n")
    stats.write_text("Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs\n"
                     "dsa::attend_gather_kernel(int),2,2000,1000,90,1000,1000\n"
                     "dsa::topk_seg_kernel<1024,16384>(float),1,200,200,10,200,200\n")
    text = ps.mfma(str(counters), str(stats), "cmd c", "cmd t")
    rows = [l.split() for l in text.splitlines() if not l.startswith("#")]
    # 1228800 busy cycles over 1 us at 2.4 GHz on 1024 SIMDs = 0.5 of the chip
    assert rows == [["dsa::attend_gather_kernel", "1000", "1228800", "1.00", "0.500"]]


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_work_decode_closed_form():
    # decode config: every visible pair and every selected key counted once
    inp = dict(B=2, Tq=1, Tk=1000, Hi=4, d=8, H=3, kd=16, vd=8, top_k=100, dtype="bf16")
    w = bench.algorithmic_work(inp)
    idx_bytes = 2 * 1000 * 8 * 2 + 2 * 4 * 8 * 2 + 2 * 4 * 4 + 2 * 1000 * 4
    assert w["index"] == (idx_bytes, 2 * 4 * 8 * 2 * 1000)
    assert w["topk"] == (2 * 1000 * 4 + 2 * 100 * 4, 0)
    att_bytes = 2 * 100 * 16 * 2 + 2 * 3 * 16 * 2 + 2 * 100 * 4 + 2 * 3 * (8 + 1) * 4
    assert w["attend"] == (att_bytes, 2 * 3 * (16 + 8) * 2 * 100)
