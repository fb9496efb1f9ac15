// Internal helpers shared by the host codec and the decode launcher of libdf11.
#pragma once

#include <stdint.h>

namespace df11_internal {

// 256-entry tables in the 8-bit hierarchy for this code (root included).
int count_tables(const uint8_t *len, const uint32_t *code);

// The device table image is the 8-bit tables (n_tables x 256 uint16), then
// the multi-code decode table the kernel indexes with the next
// kDecodeTableBits stream bits: per window, {the total length of the codes
// it covers | their number << 16, their symbols one per byte}.
constexpr uint32_t kDecodeTableBits = 11;
constexpr uint32_t kDecodeTableEntries = 1u << kDecodeTableBits;
constexpr uint32_t kDecodeTableBytes = kDecodeTableEntries * 8;

// Bytes of the device table image for n_tables tables.
uint64_t lut_image_bytes(uint32_t n_tables);

}  // namespace df11_internal
