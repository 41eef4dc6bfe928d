"""The randomised ensembles run against single gfx950 instructions: format,
instruction shape, sampling strategy and exponent limits (a, b, c), after
"Accurate Models of AMD Matrix Cores", Section 5.1 (exponent-mantissa sampling
over the normal range and over the subnormal range of each input format) and
Section 5.2 (independent bit sampling).  The pages' limits are for CDNA1-3 and
FNUZ fp8; here they are the OCP formats' own ranges: E4M3 normal exponents
-6 .. 7 (2^8 * 1.875 would be the NaN code), E5M2 -14 .. 15; bf16 products are
kept below the binary32 overflow threshold with a, b exponents up to 60, and c
up to 2^120.  For independent bit sampling the last field is the largest
unbiased exponent kept (None: every finite code)."""
CASES = {
    "bf16_16_em": ("bf16", 16, "em", ((-126, 60), (-126, 60), (-126, 120))),
    "bf16_32_em": ("bf16", 32, "em", ((-126, 60), (-126, 60), (-126, 120))),
    "bf16_16_sub": ("bf16", 16, "em", ((-133, -126), (-133, -126), (-149, -126))),
    "bf16_16_bits": ("bf16", 16, "bits", 60),
    "f16_16_em": ("f16", 16, "em", ((-14, 15), (-14, 15), (-126, 120))),
    "f16_32_em": ("f16", 32, "em", ((-14, 15), (-14, 15), (-126, 120))),
    "f16_16_sub": ("f16", 16, "em", ((-24, -14), (-24, -14), (-149, -126))),
    "f16_16_bits": ("f16", 16, "bits", None),
    "e4m3_16_em": ("e4m3", 16, "em", ((-6, 7), (-6, 7), (-126, 120))),
    "e4m3_32_em": ("e4m3", 32, "em", ((-6, 7), (-6, 7), (-126, 120))),
    "e4m3_16_sub": ("e4m3", 16, "em", ((-9, -6), (-9, -6), (-149, -126))),
    "e4m3_16_bits": ("e4m3", 16, "bits", None),
    "e5m2_16_em": ("e5m2", 16, "em", ((-14, 15), (-14, 15), (-126, 120))),
    "e5m2_32_em": ("e5m2", 32, "em", ((-14, 15), (-14, 15), (-126, 120))),
    "e5m2_16_sub": ("e5m2", 16, "em", ((-16, -14), (-16, -14), (-149, -126))),
    "e5m2_16_bits": ("e5m2", 16, "bits", None),
}
