// Internal helpers shared by the planner and the kernel launchers.
#pragma once
#include <cstddef>
#include <cstdint>

#include "libra.h"

namespace libra {

// Query columns (positions x heads) per forward work item and per dQ work
// item: 32 per wave of the forward's twelve and of the dQ kernel's eight waves.
constexpr int kFwdItemColumns = 384;
constexpr int kDqItemColumns = 256;
// Keys per dK/dV work item: the dK/dV kernel's six key groups of 32 keys.
constexpr int kKvItemKeys = 192;
// Query rows per step of the dK/dV kernel: a step runs one query block of
// this many rows (from the item's first key rounded down to a multiple of
// it, to the end of its last key's sample) against all of the item's keys.
constexpr int kKvQueryBlock = 64;
// Query positions per wave, and keys per block, of the forward and dQ kernels:
// a wave computes whole blocks of kKeyBlock keys for its kQueryTile queries.
constexpr int kQueryTile = 32;
constexpr int kKeyBlock = 64;

// Checksum stored in libra_plan_info::checksum (computed with that field as 0).
uint64_t plan_checksum(const void *plan, size_t bytes);

// Copy the header of a host plan and check its magic and version.
libra_status plan_header(const void *plan, libra_plan_info *out);

// Check a host plan whose extent is the size its own header gives: magic,
// version, section bounds and alignment, checksum (about 0.2 ms for the 3 MB
// plan of a 256K-token pack); on success copy the header to *out.
libra_status plan_validate(const void *plan, libra_plan_info *out);

}  // namespace libra

namespace libra {

bool misaligned(const void *p, uintptr_t a);

// Clear the calling thread's pending HIP error before a launch, so that the
// status taken after it belongs to that launch alone.
void clear_hip_error();

// LIBRA_OK if the launches since clear_hip_error() were accepted; otherwise
// remember the HIP error for libra_last_hip_error() and return LIBRA_EHIP.
libra_status launch_status();

}  // namespace libra
