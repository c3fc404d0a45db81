"""MI355X-native paged attention over a position-agnostic KV cache with
deferred RoPE / ALiBi (the hot path of LazyAttention).

The computation lives in ``liblazyattn.so`` (hand-written HIP for gfx950,
C ABI in ``include/lazy_attn.h``); ``lazy_attn`` is its ctypes binding,
``paging`` the host block pool / document cache, ``engine`` the device state
that sequences kv-write, prefill and decode calls.
"""

from . import lazy_attn, paging  # noqa: F401
