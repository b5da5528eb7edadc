"""KV-cache byte counts.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[P1] "The Bottleneck: Why Standard MoE Inference Stalls" gives the size of the cache per token
as 2 x L x H x D x precision bytes (L layers, H KV heads, D head dimension, the factor 2 for K
and V).  For a quantized cache the plain analogue replaces "precision" by the stored bytes per
row (codes + per-group metadata) and adds the outlier records at (value bytes + 4-byte index)
each.  [P4] "The Twin Bottlenecks" writes the KV traffic term without a bytes-per-element
factor; the factor of the size formula is restored here.  A row's packed codes occupy whole
bytes: D x bits / 8 rounded up (exact for the 128-channel heads of the kernels).
"""

BYTES_PER_ROW = {  # D = head dimension, g = group size
    "fp16": lambda D, g: 2 * D,
    "bf16": lambda D, g: 2 * D,
    "int4": lambda D, g: -(-D // 2) + (D // g) * 4,   # codes + fp16 scale and zero per group
    "fp4": lambda D, g: -(-D // 2) + (D // g) * 1,    # codes + E4M3 scale per group
    "c2": lambda D, g: -(-D // 4) + (D // g) * 8,     # codes + 4 fp16 centroids per group
    "fp8row": lambda D, g: D + 4,                 # codes + fp32 scale per row
    "u2": lambda D, g: -(-D // 4) + (D // g) * 8,     # uniform 2-bit: stored like c2
    "int4s": lambda D, g: -(-D // 2) + (D // g) * 4,  # symmetric INT4: stored like int4
    "int3": lambda D, g: -(-3 * D // 8) + (D // g) * 4,  # 3-bit codes + fp16 scale and zero per group
}
OUTLIER_VALUE_BYTES = {"none": 0, "fp16": 2, "e4m3": 1}


def kv_bytes(fmt: str, L: int, H: int, D: int, tokens: int, group: int = 0,
             num_outliers: int = 0, outlier: str = "none") -> int:
    """Bytes of K and V for ``tokens`` tokens over ``L`` layers and ``H`` KV heads."""
    per_row = BYTES_PER_ROW[fmt](D, group)
    return 2 * L * H * tokens * per_row + num_outliers * (OUTLIER_VALUE_BYTES[outlier] + 4)
