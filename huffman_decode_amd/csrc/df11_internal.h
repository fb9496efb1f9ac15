// Internal helpers shared by the host codec and the decode launcher of libdf11.
#pragma once

#include <stdint.h>

namespace df11_internal {

// 256-entry tables in the 8-bit hierarchy for this code (root included).
int count_tables(const uint8_t *len, const uint32_t *code);

// Bytes of the device table image for n_tables tables.
uint64_t lut_image_bytes(uint32_t n_tables);

}  // namespace df11_internal
