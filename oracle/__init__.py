"""fp64 CPU oracle (test infrastructure only; never used by the library's product path)."""
from .sparse3d_oracle import *  # noqa: F401,F403
from .sparse3d_oracle import (LN64, Layout, dense_attend, kmax_for, layer, member_rows,
                              query_rows, select_tiles, select_topk, sparse_attend,
                              special_rows, subsample_keys, subsample_positions, tile_pool,
                              tile_scores, key_rows_dense)
