"""libqlora: frozen int8 / 4-bit weight + trainable LoRA linear on MI355X.

The computation lives in the HIP library libqlora.so (C ABI in
include/qlora.h); ``binding`` is its ctypes wrapper and ``workloads`` the
seeded synthetic inputs. Importing the package loads nothing; the first
library call does, and raises if the library has not been built.
"""

from .binding import (  # noqa: F401
    QLinear, QloraError, qlora_bwd, qlora_bwd_workspace, qlora_fwd,
    qlora_fwd_acc, qlora_fwd_workspace, qlora_quantize, qlora_quantize_rows,
    qlora_status_str, qlora_weight_bytes,
)
