"""MI355X-native splash-attention forward: block-sparse, mask-aware flash
attention whose loop structure is read from a compiled MaskInfo."""
