"""MI355X-native routed-expert MoE layer over frozen 4-bit expert stacks with a
per-expert pre-activation LoRA: forward, input gradient and LoRA weight gradients
as hand-written gfx950 HIP kernels behind the C ABI in include/e4b.h."""
from ._lib import E4BError, get_stats, lib, reset_stats, timing_enable, timing_read, version  # noqa: F401
from .layer import LoRA, MoELayer, QStack, route, router_bwd, router_topk  # noqa: F401
