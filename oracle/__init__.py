"""Float64 CPU oracle (test infrastructure only; see swa_oracle's header)."""
from .swa_oracle import *  # noqa: F401,F403
from .swa_oracle import (CacheConfig, NaiveRingCache, RingError, RollingDecodeCache, REGION_FRAME,  # noqa: F401
                         REGION_SPECIAL, frame_visibility, masked_attention, prefill,
                         head_layer_norm, rope3d, stream_replay, token_mask, window_frames)
