"""Global-KV byte ledger (context numbers; no device code).

The reading note "DeepSeek V4.1 Flash: Pushing the Limits of KV Cache
Compression" (section on the 890-byte four-bit cache) rebuilds the report's
figure from the disclosed layout: per global position 512 E2M1 values (256 B),
one 8-bit scale per 16 channels (32 B), 128 indexer-K E2M1 values (64 B) and one
8-bit scale per 32 indexer channels (4 B) = 356 B; three encoder source layers
hold half the sequence each (ratio 2) and one decoder source layer the whole
sequence, so a token costs (3/2 + 1) * 356 = 890 B (the report, abstract and
section 4.2.1, quotes 890 B/token).

By default this library stores main KV as OCP MXFP4 (E2M1 with one E8M0 scale
per 32 channels: 256 + 16 B) and indexer K as E2M1 with one E8M0 scale per row
(64 + 1 B): 337 B per position, 842.5 B per token under the same layer count.
With main KV in E2M1 + E4M3 per 16 channels and the indexer in MXFP4 (one E8M0
per 32 channels for queries and keys), it stores the layout above ("pages").
"""

LAYOUTS = {
    # name: (main values, main scales, indexer values, indexer scales) in bytes per position
    "pages": (512 // 2, 512 // 16, 128 // 2, 128 // 32),
    "mxfp4_e8m0": (512 // 2, 512 // 32, 128 // 2, 1),
}

# source layers that store global KV: three encoder Full layers at ratio 2 and
# one decoder Full layer at ratio 1 (report section 4.2.1)
SOURCE_RATIOS = (2, 2, 2, 1)


def bytes_per_position(layout="mxfp4_e8m0"):
    return sum(LAYOUTS[layout])


def bytes_per_token(layout="mxfp4_e8m0"):
    return sum(bytes_per_position(layout) / m for m in SOURCE_RATIOS)
