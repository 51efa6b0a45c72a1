"""Plain CPU oracle of the routed MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package (``routed_moe_layer_amd``)
imports, calls or links anything here; only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may use it.  The oracle shares no code, table,
constant generator or pre/post-processing with the HIP path.

What it computes follows four web pages:
  * "Cake SiTU backend" (FlashInfer docs): the whole layer -- group-16 NVFP4 input
    quantization, routing, FC1, SiTU, NVFP4 requantization, FC2, BF16 weighted
    finalization (intro paragraph), the six quant scales and the SiTU formula (section
    "Prepared weights and scales").
  * "torch_npu.npu_moe_init_routing_v2" (Ascend API reference): key-value sort, the
    gather row map, the per-expert cumsum histogram and per-row dynamic int8 quant
    (section 计算公式, steps 1-5).
  * "Nvfp4 Tensor" (TensorRT-Edge-LLM C++ API): a per-expert fp32 global scale applied
    after block dequantization (struct NVFP4Tensor description).

Readings where the pages are silent are listed per function.  Parity status: every
function here is pinned by the CPU tests in ``tests/test_oracle_*.py`` except the
absolute agreement of SiTU's transcendentals at arbitrary points, which is pinned only
through closed forms and limits (see ``oracle.layer.situ``).
"""

from .codecs import (E2M1_MAGNITUDES, e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode,
                     bf16_bits_to_f32, f64_to_bf16_bits)
from .nvfp4 import quantize_nvfp4, dequantize_nvfp4, pack_nibbles, unpack_nibbles
from .calib import (global_scale_from_amax, calibrate_layer, calibrate_tokens,
                    calibrate_weights, quantize_expert_stack)
from .routing import route, route_int8, route_v2, int8_static_quant
from .router import topk_softmax
from .layer import (situ, fc_exact, layer_forward, layer_forward_dense, token_forward,
                    expert_rows, combine,
                    calibrate_intermediate, intermediate_amax,
                    calibrate_intermediate_per_expert, intermediate_amax_per_expert,
                    expert_weights_decoded)

__all__ = [
    "E2M1_MAGNITUDES", "e2m1_decode", "e2m1_encode", "e4m3_decode", "e4m3_encode",
    "bf16_bits_to_f32", "f64_to_bf16_bits",
    "quantize_nvfp4", "dequantize_nvfp4", "pack_nibbles", "unpack_nibbles",
    "global_scale_from_amax", "calibrate_layer", "calibrate_tokens", "calibrate_weights",
    "quantize_expert_stack",
    "calibrate_intermediate", "intermediate_amax",
    "calibrate_intermediate_per_expert", "intermediate_amax_per_expert",
    "route", "route_int8", "route_v2", "int8_static_quant", "topk_softmax",
    "situ", "fc_exact", "layer_forward", "layer_forward_dense", "token_forward",
    "expert_rows", "combine",
    "expert_weights_decoded",
]
