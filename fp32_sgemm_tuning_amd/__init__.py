"""MI355X-native FP32 SGEMM (C = alpha*A*B + beta*C, row-major) for gfx950."""
