"""MI355X-native persistent decode megakernel for parallel-transformer MoE models.

The decode step runs in libmk.so (HIP, gfx950) behind the C ABI of
include/mk.h; `binding` is its thin ctypes layer. Importing the package loads
the library and fails if it has not been built.
"""
from .binding import (  # noqa: F401
    Decoder, MkConfig, MkError, make_config, MODE_MEGAKERNEL, MODE_KERNEL_PER_OP, EXPORTS, LIB_PATH,
    ORDER_SHIPPED, ORDER_QKV_FIRST, ORDER_ATTENTION_FIRST, PLACE_TUNED, PLACE_ROUND_ROBIN, PLACE_AFFINITY,
    PLACE_COST_MODEL, PLACE_RANDOM,
    DecodeService, stream_read, litmus_message_passing,
)
