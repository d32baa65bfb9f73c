"""MI355X-native batch-1 fp16 decode monokernel.

Importing the package has no side effects; the HIP library is loaded by
``decode_persistent_monokernel_amd.kie`` on first use.
"""
from .config import ModelConfig, PRESETS, preset  # noqa: F401
