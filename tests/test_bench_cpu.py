"""Host logic of bench.py: the names under which profile summaries and traffic
records are kept (a workload's name, with its rank count where that is not
the workload's default), and the command lines a summary records."""
import bench


def test_profile_names_carry_non_default_rank_counts():
    assert bench.profile_name("prime_fp32", 7) == "prime_fp32"
    assert bench.profile_name("small_batch", bench.WORKLOADS["small_batch"]["P"]) == "small_batch"
    assert bench.profile_name("small_batch", None) == "small_batch"
    for P in (3, 6, 12):
        assert bench.profile_name("small_batch", P) == f"small_batch_P{P}"


def test_recorded_commands_name_the_rank_count():
    text = bench.PROFILE_COMMANDS.format(root="out", case="small_batch_P3_ring_r0_fused", wl="small_batch",
                                         popt=" --P 3", key="ring/r0/fused", sq="SQ_WAVES")
    runs = [ln for ln in text.splitlines() if "--workload" in ln]
    assert len(runs) == 4 and all("--workload small_batch --P 3 --schedule ring/r0/fused" in ln for ln in runs)
    text = bench.PROFILE_COMMANDS.format(root="out", case="prime_fp32_ring_r0_fused", wl="prime_fp32", popt="",
                                         key="ring/r0/fused", sq="SQ_WAVES")
    assert "--P" not in text
