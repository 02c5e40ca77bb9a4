"""CPU oracle for quantized-KV decode attention (KVQuant's decode hot path).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code with the
HIP library.  Parity status of each function is listed in ``oracle/kvquant.py`` and
``oracle/codebook_fit.py``.
"""
from .kvquant import *  # noqa: F401,F403
from .kvquant import (StreamCache, attend, decode_head, dequant_keys, dequant_values,
                      key_field_channels, logit_tolerance_scale, nearest_code,
                      output_tolerance_scale, pack_key_records, pack_value_tiles, qk_logits,
                      quantize_keys, quantize_stream, quantize_values, rope, rope_frequencies,
                      select_outliers, softmax, unpack_key_records, unpack_value_tiles,
                      zero_code, key_scale_from_keys, key_threshold_from_keys, exceed_budget)
from .codebook_fit import clamp_inputs, finalize, fit_codebook, fit_init, fit_step, fixed_point, quantization_mse
