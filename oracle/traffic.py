"""Page-1 load-count model for a tiled matrix product (test infrastructure).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Forum comment on SRAM and GEMM tiling (item 45450456), the paragraph on what
SRAM buys a GEMM: with A and B split into T tiles each, every A tile is loaded
once and, for each A tile, every B tile is loaded, so T + T*T tile loads move
(T + T*T) * tile_size bytes.  The comment's worked numbers (T = 25 tiles of
40 MiB, and T = 13 tiles of 80 MiB after doubling the SRAM) are pinned in
tests/golden/gemm_tiling_traffic.txt.  Attention's K/V stream has the same
shape: every query tile re-reads the key/value tiles it needs, so traffic falls
as the query tile grows.
"""


def tiled_gemm_reads(tiles, tile_mib):
    """Return (tile loads, MiB read) for T = `tiles` tiles of `tile_mib` MiB."""
    loads = tiles + tiles * tiles
    return loads, loads * tile_mib
