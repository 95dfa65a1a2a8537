"""Plain fp64 CPU oracle for the causal MLA attention core (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package. The library under ``attention_mla_causal_amd`` never imports it, and
this package imports nothing from the library.
"""

from .mla_oracle import (  # noqa: F401
    QK_NOPE_HEAD_DIM,
    QK_ROPE_HEAD_DIM,
    V_HEAD_DIM,
    Q_HEAD_DIM,
    bf16_bits_to_f64,
    causal_mask_4d,
    attention_probs,
    mla_attention,
    mla_attention_rows,
)
from .mla_latent import (  # noqa: F401
    KV_LORA_RANK,
    KV_B_PER_HEAD,
    decompress_kv,
    mla_decode_latent,
    mla_decode_latent_rows,
)
from .mla_varlen import (  # noqa: F401
    mla_decode_varlen,
    mla_decode_varlen_rows,
)
from .mla_paged import (  # noqa: F401
    append_rows,
    gather_sequence,
    mla_decode_paged,
)
from .mla_prefill_varlen import mla_prefill_varlen  # noqa: F401
from .mla_masked import mla_attention_masked, visible_keys  # noqa: F401
from .mla_rope import (  # noqa: F401
    KIMI_K2_ROPE,
    ROPE_DIM,
    apply_rope,
    rope_cos_sin,
    rope_positions,
    yarn_inv_freq,
)
