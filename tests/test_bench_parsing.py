"""bench.py's reading of the library's kernel names: which expert product (and
whether with e4m3 activations) a profiled GEMM instance is.  The counter and
trace summaries pick their kernels this way, so a renamed or re-templated
kernel must still land on the right product."""
import bench


def test_eight_wave_prefill_kernel():
    assert bench.gemm_kernel_stage("void sfl::grouped_gemm_bf16_w8_kernel<0>(sfl::GemmArgs)") == ("expert_up", False)
    assert bench.gemm_kernel_stage("sfl::grouped_gemm_bf16_w8_kernel<1>") == ("expert_down", False)


def test_general_kernel_instances():
    w8a16_up = "sfl::grouped_gemm_bf16_kernel<128, 512, 64, 2, 4, 3, true, 0, -4, 32, false, true>"
    w8a8_down = "sfl::grouped_gemm_bf16_kernel<128, 256, 128, 2, 4, 3, true, 1, -4, 32, true, false>"
    decode_up = "sfl::grouped_gemm_bf16_kernel<16, 64, 128, 1, 4, 3, false, 0, 1, 16, false, true>"
    assert bench.gemm_kernel_stage(w8a16_up) == ("expert_up", False)
    assert bench.gemm_kernel_stage(w8a8_down) == ("expert_down", True)
    assert bench.gemm_kernel_stage(decode_up) == ("expert_up", False)


def test_kernels_that_are_not_an_expert_product():
    # split-K reductions, the router's score GEMM (float32 epilogue), other kernels
    assert bench.gemm_kernel_stage(
        "sfl::grouped_gemm_fixup_kernel<256, 256, 64, 2, 4, 2, false, 0, -8, 32, false>") is None
    assert bench.gemm_kernel_stage(
        "sfl::grouped_gemm_bf16_kernel<64, 64, 64, 2, 2, 3, false, 2, 8, 16, false, false>") is None
    assert bench.gemm_kernel_stage("sfl::combine_kernel<256, true, false>") is None
    assert bench.gemm_kernel_stage("sfl::grouped_gemm_f32_kernel<0>") is None
