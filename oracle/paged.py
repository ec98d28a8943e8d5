"""A KV cache held in fixed-size blocks through a block table -- TEST
INFRASTRUCTURE ONLY.

Page "推测解码与 EAGLE-3", section "KV cache 回滚", names vLLM and TensorRT-LLM
as the systems that commit a verify pass's KV on acceptance; they keep the
cache in blocks.  The pages do not describe the layout, so this is a reading
(listed in the design notes): each layer has a pool of physical blocks
[num_blocks][Hkv][block_size][d], and sequence b's logical row r lives in
physical block table[b][r // block_size] at row r % block_size.  A paged
operation is the contiguous operation on the logical view: gather the
sequence's logical rows, apply the existing oracle function, write the rows
back.

Parity: pinned (tests/test_oracle_paged.py) by a block table worked by hand
(every logical row located by reading the pool by eye), the identity table
equal to a reshape of the pool, round trips through random tables, and
writes that touch no block outside the rows written.
"""
import numpy as np


def logical_rows(pool, table_row, block_size, rows):
    """Logical rows 0..rows-1 of one sequence: [Hkv][rows][d] (a copy).

    pool: [num_blocks][Hkv][block_size][d]; table_row: the sequence's block
    ids, one per logical block.
    """
    pool = np.asarray(pool)
    out = np.empty((pool.shape[1], rows, pool.shape[3]), dtype=pool.dtype)
    for r in range(rows):
        out[:, r] = pool[int(table_row[r // block_size]), :, r % block_size]
    return out


def write_rows(pool, table_row, block_size, cache, first, last):
    """Pool with logical rows [first, last) of one sequence replaced by
    cache[:, first:last] (cache: [Hkv][>= last][d], the logical view)."""
    pool = np.array(pool, copy=True)
    for r in range(first, last):
        pool[int(table_row[r // block_size]), :, r % block_size] = cache[:, r]
    return pool


def blocks_valid(table_row, block_size, rows, num_blocks):
    """True when every block holding logical rows 0..rows-1 exists."""
    nb = (rows + block_size - 1) // block_size
    if nb > len(table_row):
        return False
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    return bool(((ids >= 0) & (ids < num_blocks)).all())
