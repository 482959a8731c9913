"""Host logic of bench.py (CPU): the algorithmic flop count of each workload,
the one-GPU refusal, and the kernel-name mapping of the profile summaries."""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# GFLOP of one rank's layer shard forward + backward (3 x the forward's
# contraction flops; causal attention over visible pairs only) and of the
# loss forward + backward (6 x rows x V_r x h; the BERT workload's loss rows
# only), worked out by hand from each workload's shapes.
EXPECTED_GF = {
    "tiny_f32_t2": (0.629, 0.805),       # per rank
    "gpt2_355m_t1": (670.1, 2577.0),
    "gpt_8p3b_t8": (357.6, 483.2),
    "bert_3p9b_t4": (998.6, 154.6),
    "gpt_175b_t8": (2821.8, 966.4),
}


@pytest.mark.parametrize("name", sorted(EXPECTED_GF))
def test_step_flops(name):
    cfg = synth.get_config(name)
    f = bench.step_flops(cfg, 1)
    layer, xent = EXPECTED_GF[name]
    assert f["layer"] / 1e9 == pytest.approx(layer, rel=1e-3)
    assert f["xent"] / 1e9 == pytest.approx(xent, rel=1e-3)
    assert f["total"] == f["layer"] + f["xent"]
    both = bench.step_flops(cfg, 2)
    assert both["layer"] == 2 * f["layer"] and both["xent"] == 2 * f["xent"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


@pytest.mark.parametrize("kernel,family", [
    ("_ZN3tpl12_GLOBAL__N_116gemm_bf16_kernelILi128ELi128ELi2ELi2ELb1ELb0ELb0ELi0EDF16bEEvNS0_4ArgsE", "gemm_nn"),
    ("void tpl::(anonymous namespace)::gemm_bf16_kernel<256, 256, 2, 4, false, false, false, 0, float>(tpl::(an",
     "gemm_tn"),
    ("_ZN3tpl12_GLOBAL__N_116gemm_bf16_kernelILi256ELi192ELi4ELi2ELb1ELb1ELb1ELi1EDF16bEEvNS0_4ArgsE", "gemm_nt"),
    ("_ZN3tpl12_GLOBAL__N_114gemm_ms_kernelILi256ELi256ELi2ELi4ELi4ELi2ELi4EDF16bEEvNS0_4ArgsE", "gemm_nt"),
    ("tpl::(anonymous namespace)::splitk_sum_kernel(float*, long, float const*, int, int, int)", "gemm_tn"),
    ("void tpl::(anonymous namespace)::attn_bwd_dkdv_bf16_kernel<64, true, 1, 4>(tpl::(anonymous namespace)::Args)",
     "attn_bwd_dkdv"),
    ("_ZN3tpl12_GLOBAL__N_120attn_bwd_pair_kernelILi96ELb1ELi2ELi2EEEvNS0_4ArgsEii", "attn_bwd_pair"),
    ("_ZN3tpl12_GLOBAL__N_119xent_dlogits_kernelIDF16bEEvPT_ilPKilPKhPKfS9_f", "xent_dlogits"),
    ("_ZN3tpl12_GLOBAL__N_118ln_fwd_wide_kernelIDF16bLi8EEEvPKT_S4_S4_PS2_PfS6_if", "layernorm_fwd"),
    ("tpl::(anonymous namespace)::embed_sort_lds_kernel(int const*, int, long, int, int, int, unsigned int*, unsig",
     "embedding_sort"),
])
def test_kernel_family(kernel, family):
    assert bench.kernel_family(kernel) == family


def test_trace_command_names_the_workload():
    assert bench.DEFAULT_WORKLOAD == "gpt_175b_t8"
    assert "bench.py --config gpt2_355m_t1 --steps 5" in bench.trace_cmd("gpt2_355m_t1")
    cmd = bench.trace_cmd("gpt_175b_t8")
    assert "bench.py --config gpt_175b_t8 --steps 5" in cmd and cmd.startswith("cd /tmp && rocprofv3 --kernel-trace")
