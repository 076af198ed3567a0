"""MoE parity cases shared by the GPU parity tests and their host-side check."""

# T, H, I, E, k, qtype, rank, zipf.  Many rows per expert: the tile MMQs,
# with experts whose last 1..32 rows past their full 64- or 128-row tiles run
# on the skinny spill launches (test_oracle_moe checks that such
# experts exist).
SPILL_CASES = [
    (512, 256, 256, 8, 2, 1, 4, 0.5),
    (640, 512, 256, 8, 2, 2, 8, 1.0),
    (330, 256, 512, 4, 4, 0, 16, 0.0),
    (1024, 256, 1024, 8, 2, 1, 4, 0.5),
    # 128-row tiles in every launch (the backward ones: 64 x 4 and 64 x 8
    # tiles) beside 27 experts of at most 8 rows: both backward spill launches
    (2048, 1024, 512, 64, 4, 0, 8, 1.0),
]
