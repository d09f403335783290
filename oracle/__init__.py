"""CPU oracle for AnchorAttention: test infrastructure, never the product path."""
from .anchor_oracle import *  # noqa: F401,F403
from .anchor_oracle import (KIND_ANCHOR, KIND_FULL, KIND_NONE, KIND_PARTIAL, allowed, backward,
                            document_ids,
                            forward, position_ids, rope, rope_theta, segment_ids, tile_plan,
                            unmasked_pairs, validate_cu)
