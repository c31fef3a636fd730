// Tile-config table lookup and default heuristic (host only).
#pragma once

#include <stdint.h>

#include "fp8w8a8.h"

namespace fp8w8a8 {

// Default heuristic for untuned shapes. Returns 0.
int default_config(int kind, int64_t N, int64_t K, int64_t M, fp8_tile_config* out);

// Table lookup (nearest M, null -> default, kill switch); 1 = table hit, 0 = default.
int lookup_config(int kind, int64_t N, int64_t K, int64_t M, fp8_tile_config* out);

// Override (or reset, with nullptr) the table directory and drop cached tables.
void set_config_dir(const char* dir);

}  // namespace fp8w8a8
