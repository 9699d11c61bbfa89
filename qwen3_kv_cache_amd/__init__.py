"""MI355X-native Qwen3-0.6B-shaped KV-cache decoder: a C-ABI HIP library
(libqdec.so) with a thin Python binding (qwen3_kv_cache_amd.qdec)."""
from . import qdec  # noqa: F401
