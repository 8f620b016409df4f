"""CPU oracle for the BitNet b1.58 BitLinear (ternary weights, int8 activations)
and for the TTQ variant (ternary weights with trained asymmetric scales).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product.
"""

from .bitlinear_oracle import (  # noqa: F401
    EPS_W,
    EPS_X,
    bf16_bits_to_f64,
    bf16_round,
    absmean_gamma,
    ternary_codes,
    k_pad,
    pack_codes,
    unpack_codes,
    act_quant,
    forward_acc,
    forward_y,
    forward_y_bias,
    bias_grad,
    w_hat,
    x_hat,
    backward,
    sign1_pack,
    sign1_unpack,
    layer_fwd_bwd,
    acc_elements,
    dx_elements,
    dw_elements,
    y_elements,
)
from .ttq_oracle import (  # noqa: F401
    ttq_init,
    ttq_codes,
    ttq_values,
    ttq_forward,
    ttq_backward,
    ttq_layer,
    ttq_y_elements,
    ttq_dx_elements,
    ttq_dw_elements,
)
