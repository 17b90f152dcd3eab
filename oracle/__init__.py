"""CPU oracle for the BitLinear forward pass (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package; the product path never imports it.
"""

from .bitlinear_oracle import (  # noqa: F401
    absmean_exact,
    act_quant,
    add_bf16,
    bf16_to_f32,
    contract,
    contract_loops,
    dequant,
    export_bf16,
    f32_to_bf16,
    forward,
    forward_acc,
    pack,
    pack_weights,
    ternarize,
    tile,
    unpack,
    untile,
    weight_quant,
    weight_scale,
)
