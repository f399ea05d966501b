// Byte sizes of the buffer resources the GEMM kernels build for one 32-row
// group of an operand.  Plain constexpr arithmetic (callable from device code
// and from a host-only unit test): a resource's size is a 32-bit byte count,
// so it must never be formed from the operand's full row count.
#pragma once

#include <stdint.h>

namespace lb {

// Rows one group of a GEMM operand covers.
constexpr int kGroupRows = 32;

// Largest K (elements per row) whose 32-row group still has a byte size and
// per-lane offsets below 2^32: 32 rows x K x 2 bytes < 2^32.
constexpr int64_t kMaxGroupK = (int64_t{1} << 26) - 1;

// Bytes a group starting at `first_row` (>= 0) of an operand with `rows`
// rows of `row_bytes` bytes may read: at most its own 32 rows, none past the
// operand's last row, zero when the group starts past the end.  32-bit
// arithmetic on purpose: in a kernel the operands are wave-uniform and must
// stay on the scalar unit (a 64-bit comparison would move them to vector
// registers and every buffer load that uses the size into a read-first-lane
// loop).
constexpr uint32_t group_bytes(int32_t rows, int32_t first_row, uint32_t row_bytes) {
  const int32_t left = rows - first_row;
  return left > 0 ? static_cast<uint32_t>(left < kGroupRows ? left : kGroupRows) * row_bytes : 0u;
}

}  // namespace lb
