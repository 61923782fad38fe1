"""block_quantized_gemv_q8_amd: block-quantized GEMV on AMD Instinct MI355X.

The compute lives in libbq8.so (hand-written HIP kernels for gfx950, C ABI
in include/bq8.h); ``api`` is its thin torch binding, loaded on first use so
that ``synth`` (seeded inputs) imports without torch or a GPU.
"""
from . import synth

_API_NAMES = {
    "Bq8Error", "lib", "status_string", "abi_version", "q8_1_quantize", "q4_0_mmvq",
    *[f"q4_0_mmvq_m{m}" for m in range(1, 18)], "q6k_pack_bytes", "q6k_pack_expand",
    "q6k_lmhead_top1_scratch_bytes", "q6k_lmhead_top1", "q6k_lmhead_candidate_max",
    "q6k_lmhead_top1_noalloc",
    "q6k_compact_bytes", "q6k_pack_compact",
    "silu_mul_q8_1", "rms_norm_q8_1",
    "q4_0_pack_bytes", "q4_0_pack", "q4_0_mmvq_packed", "q4_0_mmvq_packed_ws_bytes",
    "q4_0_mmvq_packed_workspace", "q4_0_gate_up_silu_q8_1_packed",
    "q4_0_mmvq_packed_split", "q4_0_mmvq_packed_splits", "q4_0_mmvq_packed_splits_rows",
    "rms_norm_q8_1_sum",
    "q4_0_ffn_stream_layout", "q4_0_ffn_stream", "stream_weight_table", "stream_stages",
    "hbm_read_probe",
}


def __getattr__(name):
    if name in _API_NAMES:
        from . import api

        return getattr(api, name)
    raise AttributeError(name)
