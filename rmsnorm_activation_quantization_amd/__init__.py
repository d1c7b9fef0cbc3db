"""MI355X (gfx950) fused residual-add -> RMSNorm -> activation quantization."""
